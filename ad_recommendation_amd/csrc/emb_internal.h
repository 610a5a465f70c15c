// Internal declarations shared by the host runtime (emb_host.cpp) and the gfx950 kernels
// (emb_kernels.hip).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <string>
#include <vector>

namespace emb {

constexpr uint64_t kEmpty = ~0ull;             // free-slot marker in the key buckets
constexpr int kKeysPerBucket = 15;             // 15 keys + 1 metadata word = one 128-byte line
constexpr int kWordsPerBucket = 16;
constexpr uint32_t kMiss = 0xFFFFFFFFu;
constexpr uint64_t kMix = 0x9E3779B97F4A7C15ull;  // floor(2^64 / golden ratio)
constexpr int kMaxFields = 65535;
constexpr int kMaxDim = 256;
// Probe statistics are added per block into one of kStatSlots partial slots in the arena (so that
// the blocks of a launch do not all contend for one counter) and summed by a one-block kernel.
constexpr int kStatSlots = 4096;

// 64-bit key mix used to place keys; every step is invertible.
__host__ __device__ inline uint64_t mix64(uint64_t x) {
  x = (x ^ (x >> 32)) * kMix;
  x = (x ^ (x >> 32)) * kMix;
  return x ^ (x >> 32);
}
// Multiply-shift range reduction of the high hash half onto [0, n_home).
__host__ __device__ inline uint32_t home_slot(uint64_t h, uint32_t n_home) {
  return (uint32_t)(((h >> 32) * (uint64_t)n_home) >> 32);
}

// One sub-table as the kernels see it.
struct DevTab {
  const uint64_t* buckets;  // n_buckets * 16 words; word 15 holds the rowref prefix of the bucket
  uint32_t n_home;
  uint32_t n_buckets;
};

// Everything a kernel needs to reach the flashed table.
struct DevDesc {
  DevTab tab[2];
  int32_t n_tables;
  int32_t n_fields;
  int32_t granule;     // row elements per rowref unit
  int32_t var_dim;     // 1 when field widths differ
  int32_t fixed_dim;   // the common width when var_dim == 0
  int32_t max_dim;     // widest field
  int32_t out_width;   // sum of field widths = pooled output / gradient row width
  int32_t row_f16;
  int32_t has_master;
  void* rows;
  float* acc;
  float* master;
  float* linear;         // FTRL linear state z (null unless the table keeps it)
  const int32_t* fdim;   // [F] width per field
  const int32_t* fcol;   // [F] first pooled column per field
  const int32_t* fgran;  // [F] rowref units per row of the field
  uint32_t rowref_space; // rowref values are < rowref_space
  uint32_t fdiv_m;       // n / n_fields == (n * fdiv_m) >> fdiv_s for every n < 2^31
  int32_t fdiv_s;
  // Width classes (mixed-width tables): the backward sorts by (class, rowref), the class being
  // log2 of the lanes a row of the field takes, so that each update piece sees one row width.
  int32_t classed;       // 1: sort keys carry the class above bit cls_shift
  int32_t cls_shift;     // bits of the rowref part of a sort key
  const int32_t* fgsl;   // [F] class (log2 lanes per row) of each field
  uint32_t* touched;     // null, or one bit per rowref unit set when the row is updated
  unsigned long long* pstat;  // [kStatSlots][4] partial probe statistics, zero between launches
};

// End-of-PASS write-back of the rows touched since the last flash: the bitmap is read in blocks
// of kWbWords words; count, scan and gather run over a range of those blocks at a time.
constexpr int kWbWords = 1024;
struct WbLaunch {
  uint32_t* touched;     // the bitmap (cleared as it is gathered)
  int64_t n_words;
  int32_t granule;
  int32_t row_bytes;     // bytes of one rowref unit of rows (granule * element size)
  int32_t has_master;
  const uint8_t* rows;
  const float* acc;
  const float* master;
  const float* linear;   // FTRL linear state, or null
  uint32_t* bcount;      // [blocks + 1] set bits per block, then their exclusive prefix and total
  int64_t blocks;
  // gather over blocks [b0, b1): outputs at index (prefix - base)
  int64_t b0, b1;
  uint32_t base;
  uint32_t* out_unit;
  uint8_t* out_rows;
  float* out_acc;
  float* out_master;
  float* out_linear;
};
hipError_t launch_wb_count(const WbLaunch& a, hipStream_t st);   // bcount = per-block counts
hipError_t launch_wb_scan(const WbLaunch& a, hipStream_t st);    // bcount -> exclusive prefix
hipError_t launch_wb_gather(const WbLaunch& a, hipStream_t st);  // compact blocks [b0, b1)

// Kernel timing: events bracket each launch when enabled.
struct Timing {
  bool on = false;
  std::string only;  // empty = every kernel
  struct Rec {
    const char* name;
    hipEvent_t a, b;
  };
  std::vector<Rec> pool;
  size_t used = 0;
};

struct LaunchCtx {
  hipStream_t stream;
  Timing* timing;
};

// Claims a start/stop event pair for one kernel launch when timing is on (r stays null
// otherwise); the launch records them around the dispatch.
struct KTimer {
  LaunchCtx& c;
  Timing::Rec* r = nullptr;
  KTimer(LaunchCtx& ctx, const char* name);
};

struct FwdLaunch {
  DevDesc d;
  const int64_t* keys;
  const int32_t* offsets;
  int32_t n_bags;
  int32_t nnz;
  void* out;
  int32_t out_f16;
  uint32_t* rowref;
  int64_t* slot;
  unsigned long long* n_miss;
  int32_t probe;  // 0: by bucket-array size, 1: wave-cooperative, 2: per-lane
  int32_t mode;   // 0: probe and pool, 1: probe only, 2: pool only (rowrefs read from `rowref`)
  // probe statistics (null: none): [0] += scans run, [1] += scans that read past the home
  // bucket, [2] += buckets read, [3] = max(buckets read by one scan)
  unsigned long long* stats;
};

// Batch validation (EMB_VALIDATE=1): offsets start at 0, never decrease and end at nnz; with
// rowrefs, each is a miss or names a whole row of its bag's field.  Bits of *flag: 1 offsets[0],
// 2 a decrease, 4 the end, 8 a rowref.
struct ValArgs {
  DevDesc d;
  const int32_t* offsets;
  int32_t n_bags;
  int32_t nnz;
  const uint32_t* rowref;  // null: offsets only
  uint32_t* flag;
};
hipError_t launch_validate(const ValArgs& a, hipStream_t st);

// The library's static backward scratch: its size in bytes, and its device address on the
// current device (looked up once per device).
size_t scratch_bytes();
hipError_t scratch_address(void** ptr);


struct BwdLaunch {
  DevDesc d;
  const uint32_t* rowref;
  const int32_t* offsets;
  int32_t n_bags;
  int32_t nnz;
  const void* grad;
  int32_t grad_f16;
  float lr, eps;
  int32_t ftrl;          // 1: FTRL-Proximal (alpha = lr), 0: Adagrad
  float beta, l1, l2;
  void* ws;
  size_t ws_bytes;
  uint32_t* unique;
  int32_t* count;
  int64_t* n_unique;
  int32_t stage;         // 0: dedup and update, 1: dedup only, 2: update of a deduped workspace
};

// Workspace carve-up for the backward (same on host and device side).
struct BwdPlan {
  int32_t n;           // items (occurrences)
  int32_t ipt;         // sort items per thread (tile = 256 * ipt)
  int32_t tiles;       // sort tiles
  int32_t passes;      // radix passes
  int32_t bits;        // digit bits per pass (<= 11); one extra bin holds misses
  int32_t gsl;         // log2 lanes per row in the update kernels
  int32_t rounds;      // occurrences per lane group in an update piece (widest rows)
  int32_t pw;          // occurrences per update piece
  int32_t n_pieces;    // update pieces
  int32_t pdim;        // floats per partial
  int32_t groups;      // histogram groups of tiles
  int32_t tile_group;  // tiles per group
  size_t off_ka, off_va, off_kb, off_vb, off_counts, off_gsum, off_tot, off_ctr, off_seg;
  size_t off_phead, off_ptail, off_pflag, off_pkey;
  size_t bytes;
};
// `classed`: sort keys carry a 3-bit width class above the rowref bits (DevDesc::classed).
BwdPlan plan_bwd(int64_t nnz, uint32_t rowref_space, int32_t max_dim, int32_t row_f16,
                 int32_t classed);

// Layout build on the device: the ordered linear-probing layout of the host builder, computed by a
// radix sort of (table offset + home, caller index), a run-local sort of equal homes by key, a
// prefix-max scan for the slots (slot_i = i + max_{j<=i}(home_j - j) within a table) and a prefix
// sum of row units for the rowrefs.
constexpr int kBuildIpt = 8;
constexpr int kBuildTile = 256 * kBuildIpt;  // items per block of the build's scans
struct BuildArgs {
  const uint64_t* keys;    // [n] keys in the caller's order
  int64_t n;
  int32_t n_tables;
  uint32_t n_home0, n_home1;
  uint32_t* skey;          // [n] sort keys: home, plus n_home0 for table 1
  uint32_t* sval;          // [n] caller indices
  uint32_t* dup;           // [1] set when two keys are equal
  const int32_t* gran;     // [F] rowref units per row of each field
  // one table's segment [s0, s1) of the sorted order
  const uint32_t* sk;      // sorted sort keys
  uint32_t* sv;            // sorted caller indices (equal homes reordered by key in place)
  int64_t s0, s1;
  uint32_t home_base;      // the table's offset inside the sort keys
  int64_t* bmax;           // [blocks + 1] per block max of (home - local index) -> exclusive prefix max
  uint32_t* bsum;          // [blocks + 1] per block row units -> exclusive prefix sum
  int64_t blocks;
  uint64_t* buckets;       // bucket words of every table
  uint64_t bucket_base, n_buckets;
  uint32_t rowref_base;
  unsigned long long* disp;  // [2] sum and max of (slot - home)
  uint64_t tail_from;      // prefix words [tail_from, n_buckets) of the table get tail_value
  uint32_t tail_value;
};
hipError_t launch_build_homes(const BuildArgs& a, hipStream_t st);
// Radix sort of (skey, sval) over key_bits bits with plan p's buffers at ws; returns the sorted
// arrays (inside ws).
hipError_t launch_build_sort(const BuildArgs& a, const BwdPlan& p, uint8_t* ws, uint32_t** ks,
                             uint32_t** vs, hipStream_t st);
hipError_t launch_build_ties(const BuildArgs& a, hipStream_t st);
hipError_t launch_build_scan(const BuildArgs& a, hipStream_t st);   // bmax, bsum and their scans
hipError_t launch_build_place(const BuildArgs& a, hipStream_t st);  // keys, prefix words, tail

// Launchers (emb_kernels.hip).  Each returns hipSuccess or the launch error.
hipError_t launch_lookup_pool(const FwdLaunch& a, LaunchCtx& ctx);
hipError_t launch_sparse_bwd(const BwdLaunch& a, const BwdPlan& p, LaunchCtx& ctx);

}  // namespace emb
