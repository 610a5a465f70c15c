// gfx950 kernels for one training step of a GPU-resident sparse embedding layer.
//
// Forward (one launch): probe each key of a CSR batch in the prebuilt, insert-free table and
// sum-pool each bag (Tencent PCG GPU training talk: unified table, one lookup kernel for all
// fields; JD ads article 4.2.1: EmbeddingBag sum pooling over ids + offsets).
//
// Backward: deduplicate the touched rows by a stable LSD radix sort of (rowref, bag) pairs, then a
// fused pass that sums each row's upstream-gradient slices and applies element-wise sparse Adagrad
// to that row only (JD ads article 3.2.1; fp16 rows with fp32 master/state, 3.2.3 and 5.2).
// Everything is memory-bound: no matrix cores, 16-byte vector loads, LDS for tile staging.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <mutex>
#include <type_traits>
#include <vector>

#include "emb_internal.h"

// Launches a kernel; when the launch is being timed, the dispatch itself carries the start and
// stop events, so the recorded span is the kernel's own execution, not the gap around it.
#define EMB_LAUNCH(tm, K, G, B, SHM, ST, ...)                                              \
  do {                                                                                      \
    if ((tm).r) hipExtLaunchKernelGGL(K, G, B, SHM, ST, (tm).r->a, (tm).r->b, 0, __VA_ARGS__); \
    else hipLaunchKernelGGL(K, G, B, SHM, ST, __VA_ARGS__);                                 \
  } while (0)

namespace emb {

namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- vector load/store as fp32
template <typename T, int N> struct VecOf;
template <> struct VecOf<float, 4> { typedef f32x4 t; };
template <> struct VecOf<float, 8> { typedef f32x8 t; };
template <> struct VecOf<_Float16, 4> { typedef f16x4 t; };
template <> struct VecOf<_Float16, 8> { typedef f16x8 t; };
template <int N> struct F32V;
template <> struct F32V<4> { typedef f32x4 t; };
template <> struct F32V<8> { typedef f32x8 t; };

template <typename T, int N>
__device__ __forceinline__ typename F32V<N>::t load_f32(const T* p) {
  typedef typename VecOf<T, N>::t V;
  V v = *reinterpret_cast<const V*>(p);
  return __builtin_convertvector(v, typename F32V<N>::t);
}
template <typename T, int N>
__device__ __forceinline__ void store_from_f32(T* p, typename F32V<N>::t x) {
  typedef typename VecOf<T, N>::t V;
  *reinterpret_cast<V*>(p) = __builtin_convertvector(x, V);
}

// Raw vector loads: every gather in a hot loop is issued unconditionally (masked-off lanes read a
// valid stand-in address) and converted only after the whole batch of loads is in flight.
template <typename T, int N>
__device__ __forceinline__ typename VecOf<T, N>::t load_raw(const T* p) {
  return *reinterpret_cast<const typename VecOf<T, N>::t*>(p);
}
template <typename T, int N>
__device__ __forceinline__ typename F32V<N>::t to_f32(typename VecOf<T, N>::t v) {
  return __builtin_convertvector(v, typename F32V<N>::t);
}

// ---------------------------------------------------------------- wave / block helpers
__device__ __forceinline__ int lane_id() { return __lane_id(); }
// Set bits of a wave-wide mask in the lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t o = __shfl_up(v, d, 64);
    if (lane_id() >= d) v += o;
  }
  return v;
}

// Exclusive scan over the 256 threads of a block; returns the thread's exclusive prefix and the
// block total.  `s_wsum` is kWaves words of LDS.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* s_wsum, uint32_t& total) {
  const int w = threadIdx.x >> 6;
  uint32_t inc = wave_incl_scan(v);
  if (lane_id() == 63) s_wsum[w] = inc;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    uint32_t s = s_wsum[i];
    pre += (i < w) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return pre + inc - v;
}

// ---------------------------------------------------------------- probe
// Both tables' descriptors as table 0's values plus table 1's differences from them.  Both
// tables' buckets lie in one array, so a bucket is also named by its index from table 0's first
// bucket.  Picking a table per lane as a select between the two tables' fields in the kernel
// argument lets the compiler turn the select into a per-lane load from the argument block, a
// memory round trip in front of every bucket read; selecting a difference or zero keeps it a
// register operation, and bucket addresses keep the global address space of table 0's pointer.
struct Tabs {
  const uint64_t* base;     // table 0's first bucket
  uint32_t dbk;             // table 1's first bucket minus table 0's, in buckets (mod 2^32)
  uint32_t nh0, dnh;        // home slots: table 0's, table 1's minus table 0's
  uint32_t nbk0, dnbk;      // buckets: likewise
  bool two;
  // bucket index from table 0's first bucket of bucket b of table t
  __device__ __forceinline__ uint32_t global_bucket(uint32_t t, uint32_t b) const {
    return b + (t ? dbk : 0u);
  }
  __device__ __forceinline__ const uint64_t* bucket(uint32_t gb) const {
    return base + (uint64_t)gb * kWordsPerBucket;
  }
};
__device__ __forceinline__ Tabs scalar_tabs(const DevDesc& d) {
  Tabs t;
  t.two = d.n_tables == 2;
  t.base = d.tab[0].buckets;
  t.nh0 = d.tab[0].n_home;
  t.nbk0 = d.tab[0].n_buckets;
  t.dbk = t.two ? (uint32_t)((d.tab[1].buckets - d.tab[0].buckets) / kWordsPerBucket) : 0u;
  t.dnh = t.two ? d.tab[1].n_home - t.nh0 : 0u;
  t.dnbk = t.two ? d.tab[1].n_buckets - t.nbk0 : 0u;
  return t;
}
// The table of a key: (key & 1) when the table is split in two, else 0.
__device__ __forceinline__ uint32_t table_of_key(const Tabs& tb, uint64_t key) {
  return (tb.two && (key & 1ull)) ? 1u : 0u;
}
struct TabSel {
  const uint64_t* buckets;
  uint32_t n_home, n_buckets;
};
__device__ __forceinline__ TabSel pick_tab(const Tabs& tb, uint64_t key) {
  const uint32_t t = table_of_key(tb, key);
  TabSel s;
  s.buckets = tb.bucket(tb.global_bucket(t, 0u));
  s.n_home = tb.nh0 + (t ? tb.dnh : 0u);
  s.n_buckets = tb.nbk0 + (t ? tb.dnbk : 0u);
  return s;
}

__device__ __forceinline__ uint32_t div_fields(const DevDesc& d, uint32_t n) {
  return (uint32_t)(((uint64_t)n * d.fdiv_m) >> d.fdiv_s);
}

// Ordered linear probing over 128-byte buckets of 15 keys: scan from the home slot until the key
// or an empty slot.  On a hit the rowref is the bucket's stored prefix plus the row units of the
// occupied slots before the hit (rows are stored in slot order).
//
// Two forms.  In the per-lane form below, one lane reads its key's whole bucket (eight 16-byte
// loads); it needs the least work per key and is the faster one while the table's buckets stay
// within the reach of the address-translation caches.
// `nread` receives the buckets the scan read (0 when no scan runs: the EMPTY key, or a key of
// another field than its bag's).
template <bool VAR>
__device__ __forceinline__ uint32_t probe_key(const DevDesc& d, const Tabs& tabs, uint64_t key,
                                              int bag_field, int64_t& slot, uint32_t& nread) {
  slot = -1;
  nread = 0;
  if (key == kEmpty || (int)(key >> 48) != bag_field) return kMiss;
  const TabSel tb = pick_tab(tabs, key);
  const uint32_t home = home_slot(mix64(key), tb.n_home);
  uint32_t b = home / (uint32_t)kKeysPerBucket;
  uint32_t l0 = home - b * (uint32_t)kKeysPerBucket;
  for (;;) {
    if (b >= tb.n_buckets) return kMiss;  // unreachable with a well-formed terminator bucket
    ++nread;
    const u64x2* wp = reinterpret_cast<const u64x2*>(tb.buckets + (uint64_t)b * kWordsPerBucket);
    u64x2 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = wp[i];
    uint32_t occ = 0, match = 0;
#pragma unroll
    for (int l = 0; l < kKeysPerBucket; ++l) {
      const uint64_t w = (l & 1) ? v[l >> 1].y : v[l >> 1].x;
      occ |= (uint32_t)(w != kEmpty) << l;
      match |= (uint32_t)(w == key) << l;
    }
    const uint32_t stop = (match | (~occ & 0x7FFFu)) & ((0x7FFFu << l0) & 0x7FFFu);
    if (stop) {
      const int l = __builtin_ctz(stop);
      if (!((match >> l) & 1u)) return kMiss;
      const uint32_t below = occ & ((1u << l) - 1u);
      uint32_t rr = (uint32_t)v[7].y;  // word 15: rowref prefix of the bucket
      if (!VAR) {
        rr += __builtin_popcount(below);
      } else {
        uint32_t gq[kKeysPerBucket];
#pragma unroll
        for (int q = 0; q < kKeysPerBucket; ++q) {
          const uint64_t w = (q & 1) ? v[q >> 1].y : v[q >> 1].x;
          gq[q] = (uint32_t)d.fgran[((below >> q) & 1u) ? (int)(w >> 48) : 0];
        }
#pragma unroll
        for (int q = 0; q < kKeysPerBucket; ++q) rr += ((below >> q) & 1u) ? gq[q] : 0u;
      }
      slot = (int64_t)b * kKeysPerBucket + l;
      return rr;
    }
    ++b;
    l0 = 0;
  }
}

// In the wave-cooperative form, the eight lanes of a lane group read one bucket together, lane s
// loading 16 bytes (slots 2s and 2s+1; lane 7's second word is the prefix), so one load
// instruction touches eight buckets instead of 64.  When the buckets span more memory than the
// translation caches reach, each of the per-lane form's eight instructions re-misses on 64 pages.
// Measured on MI355X: random 128-byte lines read by one lane each come at ~10 G lines/s against
// ~48 G lines/s read by eight lanes each.  On the 64-field, batch-131072 forward the per-lane form
// takes 3.4, 5.2 and 5.8 ms at 200M, 400M and 800M keys (3.4, 6.8 and 13.6 GB of buckets); the
// cooperative form took 2.7-2.9 ms there in its first version and takes 1.70 ms at 800M keys now
// (early next-bucket loads, each key evaluated once from ballots, table descriptors in scalar
// registers).  Below 2 GiB of buckets the per-lane form is as fast or faster: 1.31 against 1.34 ms
// on the 100-field forward (0.7 GB of buckets), 0.282 against 0.435 ms on the mixed-width 40-field
// one, whose cooperative form keeps the group evaluation.  Hence the 2 GiB switch.
struct BucketHit {
  bool stop;      // the key or an empty slot was found in this bucket
  uint32_t rr;    // rowref on a hit, kMiss otherwise
  int l;          // slot within the bucket on a hit
};

// Evaluates one bucket for the group's key `key` from the group's loaded words (this lane's
// slots 2*sub, 2*sub+1), scanning from slot l0.  Every lane of the wave must call it (it uses
// cross-lane operations); the result is uniform within each lane group.
template <bool VAR>
__device__ __forceinline__ BucketHit eval_bucket(const DevDesc& d, u64x2 v, uint64_t key, int l0,
                                                 int sub, int grp) {
  const bool last = sub == 7;  // this lane's second word is the prefix, not a slot
  const uint32_t m = (uint32_t)(v.x == key) | ((uint32_t)(!last && v.y == key) << 1);
  const uint32_t o = (uint32_t)(v.x != kEmpty) | ((uint32_t)(!last && v.y != kEmpty) << 1);
  uint32_t packed = (m << (2 * sub)) | (o << (16 + 2 * sub));
  packed |= __shfl_xor(packed, 1, 64);
  packed |= __shfl_xor(packed, 2, 64);
  packed |= __shfl_xor(packed, 4, 64);
  const uint32_t match = packed & 0x7FFFu, occ = (packed >> 16) & 0x7FFFu;
  const uint32_t prefix = (uint32_t)__shfl((unsigned long long)v.y, grp * 8 + 7, 64);
  const uint32_t stop = (match | (~occ & 0x7FFFu)) & ((0x7FFFu << l0) & 0x7FFFu);
  BucketHit h;
  h.stop = stop != 0;
  h.l = stop ? __builtin_ctz(stop) : 0;
  const bool hit = h.stop && ((match >> h.l) & 1u);
  const uint32_t below = occ & ((1u << h.l) - 1u);
  uint32_t units;
  if (!VAR) {
    units = __builtin_popcount(below);
  } else {
    // row units of the occupied slots before the hit, summed over the group's lanes
    // (the field index is selected before the table read: an empty slot's field bits are 0xFFFF)
    const bool u0 = (below >> (2 * sub)) & 1u, u1 = (below >> (2 * sub + 1)) & 1u;
    const uint32_t g0 = (uint32_t)d.fgran[u0 ? (int)(v.x >> 48) : 0];
    const uint32_t g1 = (uint32_t)d.fgran[u1 ? (int)(v.y >> 48) : 0];
    units = (u0 ? g0 : 0u) + (u1 ? g1 : 0u);
    units += __shfl_xor(units, 1, 64);
    units += __shfl_xor(units, 2, 64);
    units += __shfl_xor(units, 4, 64);
  }
  h.rr = hit ? prefix + units : kMiss;
  return h;
}

// Lanes whose second loaded word is a slot (in each group of eight, lane 7's is the prefix word).
constexpr uint64_t kSlotLanes = 0x7F7F7F7F7F7F7F7Full;

// One key's scan through one bucket from the bucket's per-slot bits, split by slot parity: bit s of
// mx / ox is slot 2s (s < 8), bit s of my / oy slot 2s + 1 (s < 7); m: holds the key, o: occupied.
// l is the first slot at or after l0 that holds the key or is empty (kKeysPerBucket if none), hit
// whether it holds the key, below the occupied slots before it.
struct BitScan {
  int l;
  bool hit;
  uint32_t below;
};
__device__ __forceinline__ BitScan scan_bits(uint32_t mx, uint32_t my, uint32_t ox, uint32_t oy,
                                             int l0) {
  const uint32_t se = (mx | ~ox) & (0xFFu << ((l0 + 1) >> 1)) & 0xFFu;
  const uint32_t so = (my | ~oy) & (0x7Fu << (l0 >> 1)) & 0x7Fu;
  const int le = se ? 2 * __builtin_ctz(se) : kKeysPerBucket;
  const int lo = so ? 2 * __builtin_ctz(so) + 1 : kKeysPerBucket;
  BitScan r;
  r.l = min(le, lo);
  r.hit = r.l < kKeysPerBucket && ((((r.l & 1) ? my : mx) >> (r.l >> 1)) & 1u);
  r.below = __builtin_popcount(ox & ((1u << ((r.l + 1) >> 1)) - 1u)) +
            __builtin_popcount(oy & ((1u << (r.l >> 1)) - 1u));
  return r;
}

// ---------------------------------------------------------------- forward: probe + sum pool
constexpr int kFwdBags = 64;     // bags per block
constexpr int kFwdKeyCap = 2048; // rowrefs staged in LDS; larger blocks re-read them from HBM/L2
// Cooperative probe: keys homed in the last kSpecLanes slots of their bucket also load the next
// bucket in the first pass, up to kSpecKeys keys per chunk of 64.  On a table at load factor 0.5
// this leaves about 8 % of chunks, instead of 86 %, with a key whose scan outruns what the first
// pass loaded, for about 19 % more bucket loads, each next to a line the pass already reads.
// Measured on the 64-field, 800M-key batch: the forward went from 2.55 to 2.42 ms.
constexpr int kSpecLanes = 3;
constexpr int kSpecKeys = 16;
// bucket arrays at least this large are probed in the wave-cooperative form
constexpr uint64_t kCoopProbeBytes = 2ull << 30;

// Gathers and sums the rows of bag jb's occurrences k0..k1 (rowrefs from `rr`), EPL elements per
// lane, four rows in flight; misses (and any rowref outside the table's rowref space) read row 0
// and are dropped.
template <typename RowT, typename RR>
__device__ __forceinline__ typename F32V<16 / sizeof(RowT)>::t pool_rows(const DevDesc& d, RR rr,
                                                                         int k0, int k1, int e0) {
  constexpr int EPL = 16 / (int)sizeof(RowT);
  typedef typename F32V<EPL>::t AccV;
  typedef typename VecOf<RowT, EPL>::t Raw;
  const RowT* rows = reinterpret_cast<const RowT*>(d.rows) + e0;
  AccV acc = 0.0f;
  for (int k = k0; k < k1; k += 4) {
    uint32_t r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) r[u] = k + u < k1 ? rr(k + u) : kMiss;
    Raw x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      x[u] = load_raw<RowT, EPL>(rows + (r[u] < d.rowref_space ? (uint64_t)r[u] * d.granule : 0ull));
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += r[u] < d.rowref_space ? to_f32<RowT, EPL>(x[u]) : AccV(0.0f);
  }
  return acc;
}

// Probe statistics of one thread: scans run, scans past the home bucket, buckets read, most
// buckets one scan read.  flush() reduces them over the wave (every lane must call it) and adds
// them to the block's four LDS counters; the STATS = false form holds and does nothing.
// (The STATS = false form keeps a runtime-guarded LDS path that never runs, since the launcher
// sends counting launches to the STATS instantiation: with it the compiler allocates the forward
// the same 94 registers, five waves per SIMD, as without statistics; an empty form made it 104.)
template <bool STATS> struct ProbeStats {
  uint32_t* s;
  bool on;
  __device__ __forceinline__ ProbeStats(uint32_t* s_, bool on_) : s(s_), on(on_) {}
  __device__ __forceinline__ void add(uint32_t nread) {
    if (on) {
      atomicAdd(&s[0], 1u);
      atomicAdd(&s[1], nread > 1 ? 1u : 0u);
      atomicAdd(&s[2], nread);
      atomicMax(&s[3], nread);
    }
  }
  __device__ __forceinline__ void flush(uint32_t*) {}
};
template <> struct ProbeStats<true> {
  uint32_t scan = 0, past = 0, read = 0, most = 0;
  __device__ __forceinline__ ProbeStats(uint32_t*, bool) {}
  __device__ __forceinline__ void add(uint32_t nread) {
    scan += 1u;
    past += nread > 1 ? 1u : 0u;
    read += nread;
    most = max(most, nread);
  }
  __device__ __forceinline__ void flush(uint32_t* s) {
    for (int o = 32; o >= 1; o >>= 1) {
      scan += __shfl_xor(scan, o, 64);
      past += __shfl_xor(past, o, 64);
      read += __shfl_xor(read, o, 64);
      most = max(most, (uint32_t)__shfl_xor(most, o, 64));
    }
    if (lane_id() == 0 && scan) {
      atomicAdd(&s[0], scan);
      atomicAdd(&s[1], past);
      atomicAdd(&s[2], read);
      atomicMax(&s[3], most);
    }
  }
};

// STATS: the instantiation that counts probe statistics (per-thread counters, reduced per wave at
// the end of the probe); the others carry none of it.
template <typename RowT, typename OutT, bool VAR, bool COOP, bool STATS>
__global__ __launch_bounds__(kBlock) void k_lookup_pool(FwdLaunch a, int gs_log2) {
  constexpr int EPL = 16 / (int)sizeof(RowT);
  typedef typename F32V<EPL>::t AccV;
  __shared__ int32_t s_off[kFwdBags + 1];
  __shared__ int32_t s_lane0[kFwdBags + 1];       // mixed widths: first packed lane of each bag
  __shared__ uint32_t s_rr[kFwdKeyCap];
  __shared__ uint64_t s_pk[kWaves][64];          // keys of the wave's chunk (EMPTY: no probe)
  __shared__ uint32_t s_pb[kWaves][64];          // their home buckets (index from table 0's first)
  __shared__ uint32_t s_pl[kWaves][64];          // home lane, table, buckets after the home one
  __shared__ int32_t s_sj[kWaves][kSpecKeys];     // chunk keys that read the next bucket early
  __shared__ int32_t s_need[kWaves][64];          // next bucket (after home) a key must read; 0: done
  __shared__ int32_t s_list[kWaves][64];          // chunk keys still unresolved, in lane order
  __shared__ uint32_t s_pref[kWaves][2][64];      // rowref prefixes of each key's home / next bucket
  __shared__ uint4 s_tab[2];                      // per table: home slots, buckets, first bucket
  __shared__ uint32_t s_miss;
  __shared__ uint32_t s_stat[4];                  // probe statistics of the block
  const int tid = threadIdx.x;
  const int32_t j0 = (int32_t)blockIdx.x * kFwdBags;
  const int nb = min(kFwdBags, a.n_bags - j0);
  // offsets are clamped into [0, nnz] so malformed input cannot reach outside the buffers
  for (int i = tid; i <= nb; i += kBlock) s_off[i] = min(max(a.offsets[j0 + i], 0), a.nnz);
  if (tid == 0) s_miss = 0;
  if (tid < 4) s_stat[tid] = 0;
  if (COOP && tid < 2) {
    const uint32_t t = a.d.n_tables == 2 ? (uint32_t)tid : 0u;
    s_tab[tid] = make_uint4(a.d.tab[t].n_home, a.d.tab[t].n_buckets,
                            (uint32_t)((a.d.tab[t].buckets - a.d.tab[0].buckets) / kWordsPerBucket), 0u);
  }
  __syncthreads();
  const int32_t base = s_off[0];
  const int32_t nk = max(s_off[nb] - base, 0);
  const bool in_lds = nk <= kFwdKeyCap;
  const int F = a.d.n_fields;
  const int f0 = (int)((uint32_t)j0 - div_fields(a.d, (uint32_t)j0) * (uint32_t)F);

  uint32_t miss = 0;
  ProbeStats<STATS> pst(s_stat, !STATS && a.stats != nullptr);
  const Tabs tabs = scalar_tabs(a.d);
  if (a.mode == 2) {
    // pool only: the rowrefs of an earlier probe launch
    if (in_lds)
      for (int i = tid; i < nk; i += kBlock) s_rr[i] = a.rowref[base + i];
  } else if (!COOP) {
    // phase 1, per-lane form: one lane per key
    for (int i = tid; i < nk; i += kBlock) {
      const int32_t pos = base + i;
      const uint64_t key = (uint64_t)a.keys[pos];
      int lo = 0, hi = nb - 1;  // last bag whose start is <= pos
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_off[mid] <= pos) lo = mid; else hi = mid - 1;
      }
      int bf = f0 + lo;
      bf = bf >= F ? bf - (int)div_fields(a.d, (uint32_t)bf) * F : bf;
      int64_t sl;
      uint32_t nread;
      const uint32_t rr = probe_key<VAR>(a.d, tabs, key, bf, sl, nread);
      miss += (rr == kMiss);
      if (nread) pst.add(nread);
      if (in_lds) s_rr[i] = rr;
      a.rowref[pos] = rr;
      if (a.slot) a.slot[pos] = sl;
    }
  } else {
    // phase 1, wave-cooperative form: each wave probes chunks of 64 keys, eight buckets per load
    // instruction
    const int w = tid >> 6, lane = lane_id(), grp = lane >> 3, sub = lane & 7;
    // this lane's key of the wave's next chunk, loaded one chunk ahead
    uint64_t knext = (w * 64 + lane < nk) ? (uint64_t)a.keys[base + w * 64 + lane] : kEmpty;
    for (int c0 = w * 64; c0 < nk; c0 += kBlock) {
      // one lane per key: its field check, hash and home bucket, staged for the lane groups
      int nspec;
      uint64_t sm;  // keys that load their next bucket early
      {
        const int i = c0 + lane;
        uint64_t key = kEmpty;  // no probe: past the block's keys, or a miss by construction
        const uint64_t kc = knext;
        if (i < nk) {
          const int32_t pos = base + i;
          key = kc;
          int lo = 0, hi = nb - 1;  // last bag whose start is <= pos
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= pos) lo = mid; else hi = mid - 1;
          }
          int bf = f0 + lo;
          bf = bf >= F ? bf - (int)div_fields(a.d, (uint32_t)bf) * F : bf;
          if ((int)(key >> 48) != bf) key = kEmpty;  // a key outside its bag's field misses
        }
        const uint32_t t = table_of_key(tabs, key);
        const uint4 tb = s_tab[t];  // home slots, buckets, first bucket of the key's table
        const uint32_t home = key == kEmpty ? 0u : home_slot(mix64(key), tb.x);
        const uint32_t b = home / (uint32_t)kKeysPerBucket;
        const uint32_t l0 = home - b * (uint32_t)kKeysPerBucket;
        const uint32_t follow = min(tb.y - 1u - b, 0xFFFFFFu);
        s_pk[w][lane] = key;
        s_pb[w][lane] = b + tb.z;
        // bits 0-2 and 7: home lane in the bucket; bit 3: table; bits 8-31: buckets that may
        // follow the home bucket (capped; far more than any probe sequence reaches)
        s_pl[w][lane] = (l0 & 7u) | ((l0 & 8u) << 4) | (t << 3) | (follow << 8);
        // keys homed in the bucket's last kSpecLanes slots also read the next bucket in the
        // first pass, the first kSpecKeys of them in lane order
        const bool spec = key != kEmpty && follow > 0u &&
                          l0 >= (uint32_t)(kKeysPerBucket - kSpecLanes);
        sm = __ballot(spec);
        const int si = lanes_below(sm);
        if (spec && si < kSpecKeys) s_sj[w][si] = lane;
        nspec = min(__popcll(sm), kSpecKeys);
        s_need[w][lane] = 0;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      // Records the result of key j of the chunk, found (or not) in bucket e after its home
      // bucket; one lane of the key's group writes.
      auto resolve = [&](int j, uint64_t key, uint32_t e, const BucketHit& h) {
        const int i = c0 + j;
        if (sub == 0 && i < nk) {
          const uint32_t rr = key == kEmpty ? kMiss : h.rr;
          miss += (rr == kMiss);
          if (key != kEmpty) pst.add(e + 1u);
          if (in_lds) s_rr[i] = rr;
          a.rowref[base + i] = rr;
          if (a.slot) {
            const uint64_t bk = (uint64_t)(s_pb[w][j] - s_tab[(s_pl[w][j] >> 3) & 1u].z) + e;
            a.slot[base + i] = rr == kMiss ? -1 : (int64_t)(bk * kKeysPerBucket) + h.l;
          }
        }
      };
      // first pass: in round r lane group g probes key r * 8 + g in its home bucket, and in
      // spec round q the next bucket of listed key q * 8 + g; every load is issued before any is
      // evaluated, and the next chunk's keys ride with them (on the 64-field, 800M-key batch,
      // loading them here took the forward from 2.89 to 2.57 ms).  A listed key whose home
      // bucket ends its scan ignores its next bucket.
      u64x2 v[8];
      {
        u64x2 vs[kSpecKeys / 8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int j = r * 8 + grp;
          const uint64_t* bp = tabs.bucket(s_pb[w][j]);
          v[r] = *reinterpret_cast<const u64x2*>(bp + 2 * sub);
        }
#pragma unroll
        for (int q = 0; q < kSpecKeys / 8; ++q) {
          const int s = q * 8 + grp;
          vs[q] = u64x2{kEmpty, kEmpty};
          if (s < nspec) {
            const int j = s_sj[w][s];
            const uint64_t* bp = tabs.bucket(s_pb[w][j] + 1u);
            vs[q] = *reinterpret_cast<const u64x2*>(bp + 2 * sub);
          }
        }
        {
          const int in = c0 + kBlock + lane;
          knext = in < nk ? (uint64_t)a.keys[base + in] : kEmpty;
        }
        // staged values are read from LDS as each round is evaluated, not held across the loads
        asm volatile("" ::: "memory");
        if constexpr (!VAR) {
          // Each round's match and occupancy bits come from four ballots (bit 8g + s: lane s of
          // group g; slots 2s and 2s + 1), and every lane keeps the byte of its own key's group,
          // so each key is evaluated once, by the lane that staged it, instead of by all eight
          // lanes of its group in every round.  The prefix words go through LDS.  pick() packs the
          // four bytes of group g: match and occupancy of its even and of its odd slots.
          auto pick = [](uint64_t mx, uint64_t my, uint64_t ox, uint64_t oy, int g) -> uint32_t {
            const int sh = 8 * g;
            return (uint32_t)((mx >> sh) & 0xFFu) | ((uint32_t)((my >> sh) & 0xFFu) << 8) |
                   ((uint32_t)((ox >> sh) & 0xFFu) << 16) | ((uint32_t)((oy >> sh) & 0xFFu) << 24);
          };
          uint32_t hb = 0;
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const int j = r * 8 + grp;
            const uint64_t key = s_pk[w][j];
            const uint64_t mx = __ballot(v[r].x == key);
            const uint64_t my = __ballot(v[r].y == key) & kSlotLanes;
            const uint64_t ox = __ballot(v[r].x != kEmpty);
            const uint64_t oy = __ballot(v[r].y != kEmpty) & kSlotLanes;
            if (sub == 7) s_pref[w][0][j] = (uint32_t)v[r].y;
            if ((lane >> 3) == r) hb = pick(mx, my, ox, oy, lane & 7);
            asm volatile("" ::: "memory");  // one round's key read at a time
          }
          // the next buckets of the listed keys: lane L, listed at si, reads group si & 7 of
          // spec round si >> 3
          const int si = lanes_below(sm);
          const bool spec = ((sm >> lane) & 1ull) && si < nspec;
          uint32_t nb = 0;
#pragma unroll
          for (int q = 0; q < kSpecKeys / 8; ++q) {
            if (q * 8 >= nspec) break;
            const int s = q * 8 + grp;
            const bool ok = s < nspec;
            const int j = ok ? s_sj[w][s] : 0;
            const uint64_t key = ok ? s_pk[w][j] : kEmpty;
            const uint64_t mx = __ballot(vs[q].x == key);
            const uint64_t my = __ballot(vs[q].y == key) & kSlotLanes;
            const uint64_t ox = __ballot(vs[q].x != kEmpty);
            const uint64_t oy = __ballot(vs[q].y != kEmpty) & kSlotLanes;
            if (sub == 7 && ok) s_pref[w][1][j] = (uint32_t)vs[q].y;
            if (spec && (si >> 3) == q) nb = pick(mx, my, ox, oy, si & 7);
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
          // one lane per key: the home bucket from its home slot, then the early next bucket
          const uint64_t key = s_pk[w][lane];
          const uint32_t pl = s_pl[w][lane];
          const uint32_t follow = pl >> 8;
          const BitScan hs = scan_bits(hb & 0xFFu, (hb >> 8) & 0xFFu, (hb >> 16) & 0xFFu, hb >> 24,
                                       (int)(pl & 7u) + (int)((pl >> 4) & 8u));
          bool done = true;
          int need = 0;
          uint32_t e = 0u, rr = kMiss;
          int l = hs.l;
          if (key == kEmpty) {
          } else if (hs.l < kKeysPerBucket) {
            if (hs.hit) rr = s_pref[w][0][lane] + hs.below;
          } else if (spec) {
            const BitScan ns =
                scan_bits(nb & 0xFFu, (nb >> 8) & 0xFFu, (nb >> 16) & 0xFFu, nb >> 24, 0);
            e = 1u;
            l = ns.l;
            if (ns.l < kKeysPerBucket) {
              if (ns.hit) rr = s_pref[w][1][lane] + ns.below;
            } else if (follow > 1u) {
              done = false;
              need = 2;
            }
          } else if (follow > 0u) {
            done = false;
            need = 1;
          }
          s_need[w][lane] = need;
          const int i = c0 + lane;
          if (done && i < nk) {
            miss += (rr == kMiss);
            if (key != kEmpty) pst.add(e + 1u);
            if (in_lds) s_rr[i] = rr;
            a.rowref[base + i] = rr;
            if (a.slot) {
              const uint64_t bk = (uint64_t)(s_pb[w][lane] - s_tab[(pl >> 3) & 1u].z) + e;
              a.slot[base + i] = rr == kMiss ? -1 : (int64_t)(bk * kKeysPerBucket) + l;
            }
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        } else {
          // mixed widths: a hit's rank sums the row units of the occupied slots before it, so
          // each group evaluates its bucket together (eval_bucket)
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const int j = r * 8 + grp;
            const uint64_t key = s_pk[w][j];
            const uint32_t pl = s_pl[w][j];
            const int l0 = (int)(pl & 7u) + (int)((pl >> 4) & 8u);
            const BucketHit h = eval_bucket<VAR>(a.d, v[r], key, l0, sub, grp);
            if (key == kEmpty || h.stop || (pl >> 8) == 0u) resolve(j, key, 0u, h);
            else if (sub == 0) s_need[w][j] = 1;
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
          for (int q = 0; q < kSpecKeys / 8; ++q) {
            if (q * 8 >= nspec) break;
            const int s = q * 8 + grp;
            const bool ok = s < nspec;
            const int j = ok ? s_sj[w][s] : 0;
            const uint64_t key = ok ? s_pk[w][j] : kEmpty;
            const uint32_t pl = s_pl[w][j];
            const int need = ok ? s_need[w][j] : 0;
            const BucketHit h = eval_bucket<VAR>(a.d, vs[q], key, 0, sub, grp);
            if (need == 1) {  // the home bucket did not end the scan
              if (h.stop || (pl >> 8) <= 1u) {
                resolve(j, key, 1u, h);
                if (sub == 0) s_need[w][j] = 0;
              } else if (sub == 0) {
                s_need[w][j] = 2;
              }
            }
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      
        }
}
      // further passes: the keys still unresolved (a few per chunk at load factor 0.5), listed
      // in lane order and probed eight per round in the next bucket each still needs
      while (true) {
        const int need = s_need[w][lane];
        const uint64_t um = __ballot(need > 0);
        if (um == 0ull) break;
        const int n = __popcll(um);
        if (need > 0) s_list[w][lanes_below(um)] = lane;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          if (r * 8 >= n) break;
          const int s = r * 8 + grp;
          v[r] = u64x2{kEmpty, kEmpty};
          if (s < n) {
            const int j = s_list[w][s];
            const uint64_t* bp = tabs.bucket(s_pb[w][j] + (uint32_t)s_need[w][j]);
            v[r] = *reinterpret_cast<const u64x2*>(bp + 2 * sub);
          }
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          if (r * 8 >= n) break;
          const int s = r * 8 + grp;
          const bool ok = s < n;
          const int j = ok ? s_list[w][s] : 0;
          const uint64_t key = ok ? s_pk[w][j] : kEmpty;
          const uint32_t pl = s_pl[w][j];
          const uint32_t e = ok ? (uint32_t)s_need[w][j] : 0u;
          const BucketHit h = eval_bucket<VAR>(a.d, v[r], key, 0, sub, grp);
          if (ok) {
            if (h.stop || e >= (pl >> 8)) {
              resolve(j, key, e, h);
              if (sub == 0) s_need[w][j] = 0;
            } else if (sub == 0) {
              s_need[w][j] = (int)e + 1;
            }
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      }
    }
  }
  if (miss) atomicAdd(&s_miss, miss);
  pst.flush(s_stat);
  __syncthreads();
  if (tid == 0 && s_miss && a.n_miss) atomicAdd(a.n_miss, (unsigned long long)s_miss);
  if (tid == 0 && a.stats && s_stat[0]) {
    unsigned long long* ps = a.d.pstat + (size_t)(blockIdx.x % (unsigned)kStatSlots) * 4u;
    atomicAdd(ps + 0, (unsigned long long)s_stat[0]);
    atomicAdd(ps + 1, (unsigned long long)s_stat[1]);
    atomicAdd(ps + 2, (unsigned long long)s_stat[2]);
    atomicMax(ps + 3, (unsigned long long)s_stat[3]);
  }
  if (a.mode == 1) return;  // probe only

  OutT* out = reinterpret_cast<OutT*>(a.out);
  if (VAR) {
    // phase 2, mixed widths: bag jb takes D/EPL consecutive lanes of a packed lane space (no
    // lane idles on a narrow field), EPL elements per lane
    if (tid < 64) {
      int L = 0;
      if (tid < nb) {
        int f = f0 + tid;
        f = f >= F ? f - (int)div_fields(a.d, (uint32_t)f) * F : f;
        L = a.d.fdim[f] / EPL;
      }
      const uint32_t incl = wave_incl_scan((uint32_t)L);
      s_lane0[tid] = (int)incl - L;
      if (tid == 63) s_lane0[64] = (int)incl;
    }
    __syncthreads();
    const int lanes = s_lane0[64];
    for (int v = tid; v < lanes; v += kBlock) {
      int lo = 0, hi = nb - 1;  // the bag whose lane range holds v
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_lane0[mid] <= v) lo = mid; else hi = mid - 1;
      }
      const int jb = lo;
      int f = f0 + jb;
      f = f >= F ? f - (int)div_fields(a.d, (uint32_t)f) * F : f;
      const int e0 = (v - s_lane0[jb]) * EPL;
      const uint32_t b = div_fields(a.d, (uint32_t)(j0 + jb));
      const int k0 = min(max(s_off[jb] - base, 0), nk), k1 = min(max(s_off[jb + 1] - base, k0), nk);
      AccV acc;
      if (in_lds)
        acc = pool_rows<RowT>(a.d, [&](int k) { return s_rr[k]; }, k0, k1, e0);
      else
        acc = pool_rows<RowT>(a.d, [&](int k) { return a.rowref[base + k]; }, k0, k1, e0);
      store_from_f32<OutT, EPL>(out + (uint64_t)b * a.d.out_width + a.d.fcol[f] + e0, acc);
    }
    return;
  }
  // phase 2: a group of 2^gs_log2 lanes per bag, EPL elements per lane
  const int lane = tid & ((1 << gs_log2) - 1);
  const int ngrp = kBlock >> gs_log2;
  const int e0 = lane * EPL;
  for (int jb = tid >> gs_log2; jb < nb; jb += ngrp) {
    int f = f0 + jb;
    f = f >= F ? f - (int)div_fields(a.d, (uint32_t)f) * F : f;
    const int D = VAR ? a.d.fdim[f] : a.d.fixed_dim;
    const int col = VAR ? a.d.fcol[f] : f * a.d.fixed_dim;
    if (e0 >= D) continue;
    const uint32_t b = div_fields(a.d, (uint32_t)(j0 + jb));
    const int k0 = min(max(s_off[jb] - base, 0), nk), k1 = min(max(s_off[jb + 1] - base, k0), nk);
    AccV acc;
    if (in_lds)
      acc = pool_rows<RowT>(a.d, [&](int k) { return s_rr[k]; }, k0, k1, e0);
    else
      acc = pool_rows<RowT>(a.d, [&](int k) { return a.rowref[base + k]; }, k0, k1, e0);
    store_from_f32<OutT, EPL>(out + (uint64_t)b * a.d.out_width + col + e0, acc);
  }
}

// ---------------------------------------------------------------- backward: radix sort
// Stable LSD radix sort of (rowref, bag) pairs.  Digits are up to 9 bits wide (see plan_bwd), as
// few passes as that allows for the row space; occurrences that missed get a bin of their own
// after every digit value, so they never widen the key and always sort last.
constexpr int kOffStage = 2048;               // bag offsets staged in LDS for the first pass
constexpr int kMaxBins = (1 << 9) + 1;
constexpr uint32_t kMissKey = 0xFFFFFFFFu;    // sorted-key value of a missed occurrence

struct SortArgs {
  const uint32_t* rowref;   // first pass source
  const int32_t* offsets;
  int32_t n_bags;
  const uint32_t* kin;
  const uint32_t* vin;
  uint32_t* kout;
  uint32_t* vout;
  uint32_t* counts;   // [tiles][bins]: each tile's digit prefix within its group of tiles
  uint32_t* gsum;     // [groups][bins]: group totals, then their exclusive prefix over groups
  uint32_t* tot;      // [bins]
  int32_t groups;     // tile groups of tile_group consecutive tiles
  int32_t tile_group;
  uint32_t* ctr;      // small counters, zeroed by the first scan
  int32_t n;
  int32_t tiles;
  int32_t tile;       // items per tile
  uint32_t rowref_space;
  int32_t shift;
  int32_t bits;       // digit bits of this pass; bin (1 << bits) holds the misses
  // width classes of mixed-width tables (the first pass puts them above the rowref bits)
  int32_t classed;
  int32_t cls_shift;
  const int32_t* fgsl;
  int32_t n_fields;
  uint32_t fdiv_m;
  int32_t fdiv_s;
};

__device__ __forceinline__ uint32_t sort_key_of(uint32_t rr, uint32_t space) {
  return rr < space ? rr : kMissKey;  // a miss, or any value outside the table
}
__device__ __forceinline__ uint32_t digit_of(uint32_t k, int shift, int bits) {
  return k == kMissKey ? (1u << bits) : ((k >> shift) & ((1u << bits) - 1u));
}

// Exclusive scan of n <= 256*E values get(i) into set(i, prefix) by one block; returns the total.
template <int E, typename Get, typename Set>
__device__ __forceinline__ uint32_t block_scan_n(int n, Get get, Set set, uint32_t* s_w) {
  const int b = threadIdx.x * E;
  uint32_t v[E], sum = 0;
#pragma unroll
  for (int u = 0; u < E; ++u) {
    v[u] = (b + u < n) ? get(b + u) : 0u;
    sum += v[u];
  }
  uint32_t total;
  uint32_t pre = block_excl_scan(sum, s_w, total);
#pragma unroll
  for (int u = 0; u < E; ++u) {
    if (b + u < n) set(b + u, pre);
    pre += v[u];
  }
  return total;
}

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2.  This maps block b
// to a logical index so that every XCD works on one contiguous range of [0, n): neighbouring
// tiles (or bins) then share cache lines in one L2.
__device__ __forceinline__ int xcd_index(int b, int n) {
  const int q = n >> 3, r = n & 7, x = b & 7, j = b >> 3;
  return x * q + min(x, r) + j;
}

// Digit histograms of a group of tile_group consecutive tiles, one tile after another: each
// tile's counts are stored as its prefix within the group, and the group's totals apart.  Each
// thread counts a run of consecutive items and adds runs of equal digits at once (sorted passes
// hold long runs of one key).  Groups map to XCDs in contiguous ranges.
template <bool FIRST>
__global__ __launch_bounds__(kBlock) void k_sort_hist(SortArgs a) {
  __shared__ uint32_t h[kMaxBins];
  __shared__ uint32_t run[kMaxBins];
  const int g = xcd_index(blockIdx.x, a.groups);
  const int bins = (1 << a.bits) + 1;
  for (int d = threadIdx.x; d < bins; d += kBlock) run[d] = 0;
  const int per = a.tile / kBlock;  // 4, 8 or 16
  const uint32_t* src = FIRST ? a.rowref : a.kin;
  const int t1 = min(a.tiles, (g + 1) * a.tile_group);
  for (int t = g * a.tile_group; t < t1; ++t) {
    for (int d = threadIdx.x; d < bins; d += kBlock) h[d] = 0;
    __syncthreads();
    const int32_t i0 = t * a.tile + (int32_t)threadIdx.x * per;
    const bool full = (int64_t)(t + 1) * a.tile <= a.n;  // every tile but possibly the last
    uint32_t k16[16];
    if (full) {
#pragma unroll
      for (int u = 0; u < 16; u += 4) {
        if (u < per) {
          const uint4 v = *reinterpret_cast<const uint4*>(src + i0 + u);
          k16[u] = v.x; k16[u + 1] = v.y; k16[u + 2] = v.z; k16[u + 3] = v.w;
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < 16; ++u) k16[u] = (u < per && i0 + u < a.n) ? src[i0 + u] : 0u;
    }
    uint32_t prev = 0xFFFFFFFFu, cnt = 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (u < per && i0 + u < a.n) {
        const uint32_t k = FIRST ? sort_key_of(k16[u], a.rowref_space) : k16[u];
        const uint32_t dg = digit_of(k, a.shift, a.bits);
        if (dg != prev) {
          if (cnt) atomicAdd(&h[prev], cnt);
          prev = dg;
          cnt = 0;
        }
        ++cnt;
      }
    }
    if (cnt) atomicAdd(&h[prev], cnt);
    __syncthreads();
    for (int d = threadIdx.x; d < bins; d += kBlock) {
      a.counts[(size_t)t * bins + d] = run[d];
      run[d] += h[d];
    }
  }
  __syncthreads();
  for (int d = threadIdx.x; d < bins; d += kBlock) a.gsum[(size_t)g * bins + d] = run[d];
}

// Exclusive scan over tile groups of each digit's group totals (one block per digit; digits map
// to XCDs in contiguous ranges so neighbouring digits share lines) and the digit totals.
__global__ __launch_bounds__(kBlock) void k_sort_scan(SortArgs a, int zero_ctr) {
  __shared__ uint32_t s_w[kWaves];
  const int bins = (1 << a.bits) + 1;
  const int d = xcd_index(blockIdx.x, bins);
  if (zero_ctr && blockIdx.x == 0 && threadIdx.x < 16) a.ctr[threadIdx.x] = 0;
  uint32_t* col = a.gsum + d;
  uint32_t carry = 0;
  for (int32_t c0 = 0; c0 < a.groups; c0 += kBlock * 4) {
    uint32_t v[4], s = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int32_t i = c0 + threadIdx.x * 4 + u;
      v[u] = i < a.groups ? col[(size_t)i * bins] : 0u;
      s += v[u];
    }
    uint32_t total;
    uint32_t pre = block_excl_scan(s, s_w, total) + carry;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int32_t i = c0 + threadIdx.x * 4 + u;
      if (i < a.groups) col[(size_t)i * bins] = pre;
      pre += v[u];
    }
    carry += total;
  }
  if (threadIdx.x == 0) a.tot[d] = carry;
}

__device__ __forceinline__ int32_t bag_search_global(const int32_t* off, int32_t lo, int32_t hi,
                                                     int32_t pos) {
  // last j in [lo, hi] with off[j] <= pos
  while (lo < hi) {
    const int32_t mid = lo + ((hi - lo + 1) >> 1);
    if (off[mid] <= pos) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Last bag j in [0, n_bags) with off[j] <= pos, found by the whole block: each round probes 256
// evenly spaced offsets and keeps the bracket containing pos (off is non-decreasing).
__device__ int32_t block_find_bag(const int32_t* off, int32_t n_bags, int32_t pos) {
  int32_t lo = 0, hi = n_bags - 1;
  while (hi - lo >= kBlock) {
    const int32_t step = (hi - lo) / kBlock + 1;
    const int32_t p = lo + (int32_t)threadIdx.x * step;
    const int c = __syncthreads_count(p <= hi && off[p] <= pos);
    const int32_t nlo = lo + (c > 0 ? c - 1 : 0) * step;
    hi = min(hi, nlo + step - 1);
    lo = nlo;
  }
  const int32_t p = lo + (int32_t)threadIdx.x;
  const int c = __syncthreads_count(p <= hi && off[p] <= pos);
  return lo + (c > 0 ? c - 1 : 0);
}

// Stable scatter of one tile by one digit.  Each wave ranks a contiguous quarter of the tile with
// ballots (one per digit bit, plus the miss bin), the tile is reordered in LDS, then written out
// in digit runs.  IPT items per thread; digits of at most LOGB bits.
template <bool FIRST, int IPT, int LOGB>
__global__ __launch_bounds__(kBlock) void k_sort_scatter(SortArgs a) {
  constexpr int TILE = kBlock * IPT;
  constexpr int BINS = (1 << LOGB) + 1;
  constexpr int E = (BINS + kBlock - 1) / kBlock;
  __shared__ uint32_t s_key[TILE];
  __shared__ uint32_t s_val[TILE];
  __shared__ uint32_t s_wcnt[kWaves][BINS];
  __shared__ uint32_t s_gbase[BINS];
  __shared__ uint32_t s_lstart[BINS];
  __shared__ uint32_t s_w[kWaves];
  __shared__ int32_t s_off[FIRST ? kOffStage + 1 : 1];

  const int tid = threadIdx.x, w = tid >> 6, lane = lane_id();
  const int t = xcd_index(blockIdx.x, a.tiles);
  const int32_t i0 = t * TILE;
  const int32_t tn = min(TILE, a.n - i0);
  const int bins = (1 << a.bits) + 1;

  // global start of each digit in this tile: all smaller digits, plus this digit in earlier tiles
  block_scan_n<E>(bins, [&](int d) { return a.tot[d]; },
                  [&](int d, uint32_t v) {
                    s_gbase[d] = v + a.gsum[(size_t)(t / a.tile_group) * bins + d] +
                                 a.counts[(size_t)t * bins + d];
                  },
                  s_w);
  for (int d = tid; d < bins; d += kBlock)
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) s_wcnt[ww][d] = 0;
  bool stage = false;
  int32_t jlo = 0, nst = 0;
  if (FIRST) {
    // bags of this tile's occurrences: stage offsets[jlo ..] in LDS when they cover the tile
    jlo = block_find_bag(a.offsets, a.n_bags, i0);
    nst = min(kOffStage + 1, a.n_bags - jlo + 1);
    for (int i = tid; i < nst; i += kBlock) s_off[i] = a.offsets[jlo + i];
    __syncthreads();
    stage = (jlo + nst - 1 == a.n_bags) || (s_off[nst - 1] > i0 + tn - 1);
  }
  __syncthreads();

  uint32_t key[IPT], val[IPT], rank[IPT];
  // all of this thread's items first (masked-off items read item 0), then the ranking
#pragma unroll
  for (int k = 0; k < IPT; ++k) {
    const int32_t li = w * (IPT * 64) + k * 64 + lane;
    const int32_t i = li < tn ? i0 + li : 0;
    key[k] = FIRST ? a.rowref[i] : a.kin[i];
    val[k] = FIRST ? 0u : a.vin[i];
  }
#pragma unroll
  for (int k = 0; k < IPT; ++k) {
    const int32_t li = w * (IPT * 64) + k * 64 + lane;  // item index inside the tile
    const bool valid = li < tn;
    const int32_t i = i0 + li;
    uint32_t kk = 0, vv = 0;
    if (valid) {
      if (FIRST) {
        kk = sort_key_of(key[k], a.rowref_space);
        if (stage) {
          int lo = 0, hi = nst - 2;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= i) lo = mid; else hi = mid - 1;
          }
          vv = (uint32_t)(jlo + lo);
        } else {
          vv = (uint32_t)bag_search_global(a.offsets, jlo, a.n_bags - 1, i);
        }
        if (a.classed && kk != kMissKey) {
          const uint32_t b = (uint32_t)(((uint64_t)vv * a.fdiv_m) >> a.fdiv_s);
          kk |= (uint32_t)a.fgsl[vv - b * (uint32_t)a.n_fields] << a.cls_shift;
        }
      } else {
        kk = key[k];
        vv = val[k];
      }
    }
    const uint32_t dg = digit_of(kk, a.shift, a.bits);
    // the lanes of this round whose item has the same digit: one ballot per digit bit (the miss
    // bin's bit included), kept as two 32-bit halves; sb is all ones where this lane's bit is set,
    // and a lane stays a peer where the ballot agrees with it
    const uint64_t vb = __ballot(valid);
    uint32_t mlo = (uint32_t)vb, mhi = (uint32_t)(vb >> 32);
#pragma unroll
    for (int bit = 0; bit <= LOGB; ++bit) {
      if (bit <= a.bits) {
        const int32_t top = (int32_t)(dg << (31 - bit));  // this bit in the sign position
        const uint64_t bb = __ballot(top < 0);
        const uint32_t sb = (uint32_t)(top >> 31);
        mlo &= ~((uint32_t)bb ^ sb);
        mhi &= ~((uint32_t)(bb >> 32) ^ sb);
      }
    }
    const uint64_t m = ((uint64_t)mhi << 32) | mlo;
    const int below = lanes_below(m);
    const uint32_t before = s_wcnt[w][dg];
    if (valid && below == 0) s_wcnt[w][dg] = before + (uint32_t)__popcll(m);
    rank[k] = before + (uint32_t)below;
    key[k] = kk;
    val[k] = vv;
  }
  __syncthreads();
  // per digit: items in earlier waves, and the digit's start inside the reordered tile
  for (int d = tid; d < bins; d += kBlock) {
    uint32_t c = 0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const uint32_t x = s_wcnt[ww][d];
      s_wcnt[ww][d] = c;
      c += x;
    }
    s_lstart[d] = c;  // per-digit tile count, scanned below
  }
  __syncthreads();
  block_scan_n<E>(bins, [&](int d) { return s_lstart[d]; },
                  [&](int d, uint32_t v) { s_lstart[d] = v; }, s_w);
  __syncthreads();
#pragma unroll
  for (int k = 0; k < IPT; ++k) {
    const int32_t li = w * (IPT * 64) + k * 64 + lane;
    if (li < tn) {
      const uint32_t dg = digit_of(key[k], a.shift, a.bits);
      const uint32_t p = s_lstart[dg] + s_wcnt[w][dg] + rank[k];
      s_key[p] = key[k];
      s_val[p] = val[k];
    }
  }
  __syncthreads();
  for (int p = tid; p < tn; p += kBlock) {
    const uint32_t kk = s_key[p];
    const uint32_t dg = digit_of(kk, a.shift, a.bits);
    const uint32_t dst = s_gbase[dg] + ((uint32_t)p - s_lstart[dg]);
    a.kout[dst] = kk;
    a.vout[dst] = s_val[p];
  }
}

// ---------------------------------------------------------------- backward: reduce + Adagrad
struct UpdArgs {
  DevDesc d;
  const uint32_t* key;   // sorted rowrefs (misses last, as kMissKey)
  const uint32_t* val;   // bag of each sorted occurrence
  int32_t n;
  uint32_t miss_key;
  const void* grad;
  float lr, eps;
  float inv_alpha, beta, l1, l2;  // FTRL: 1 / alpha (alpha = lr), beta, L1 and L2 strengths
  uint32_t* ctr;         // [1] unique-row count
  int64_t* n_unique;
  // pieces: each wave reduces `rounds` x (64 / GS) consecutive sorted occurrences
  int32_t rounds;
  int32_t pw;            // occurrences per piece
  int32_t n_pieces;
  int32_t pdim;          // floats per partial (widest row)
  float* phead;          // [n_pieces][pdim] sum of the piece's first segment when it began earlier
  float* ptail;          // [n_pieces][pdim] sum of the piece's last segment when it runs on
  uint32_t* pflag;       // [n_pieces] bit 0: tail partial; bits 1-2: head partial (1 ends here, 2 passes)
  uint32_t* pkey;        // [n_pieces][2] row and width of the tail partial's segment
};

// Row state of one lane's EPL elements as loaded: the accumulator, the weights the update reads
// (the fp32 master copy when the table keeps one, else the row itself) and, for FTRL, the linear
// state z.
template <typename RowT, int EPL, bool MASTER, bool FTRL>
struct RawState {
  typedef typename std::conditional<MASTER, float, RowT>::type WT;
  typename VecOf<float, EPL>::t acc;
  typename VecOf<WT, EPL>::t w;
};
template <typename RowT, int EPL, bool MASTER>
struct RawState<RowT, EPL, MASTER, true> {
  typedef typename std::conditional<MASTER, float, RowT>::type WT;
  typename VecOf<float, EPL>::t acc;
  typename VecOf<WT, EPL>::t w;
  typename VecOf<float, EPL>::t z;
};

// Issues the state loads of row r (row 0 stands in when `on` is false).
template <typename RowT, int EPL, bool MASTER, bool FTRL>
__device__ __forceinline__ RawState<RowT, EPL, MASTER, FTRL> load_state(const UpdArgs& a,
                                                                        uint32_t r, int e0,
                                                                        bool on) {
  typedef typename RawState<RowT, EPL, MASTER, FTRL>::WT WT;
  RawState<RowT, EPL, MASTER, FTRL> st;
  const uint64_t e = (on ? (uint64_t)r * a.d.granule : 0ull) + e0;
  st.acc = load_raw<float, EPL>(a.d.acc + e);
  st.w = MASTER ? load_raw<WT, EPL>(reinterpret_cast<const WT*>(a.d.master) + e)
                : load_raw<WT, EPL>(reinterpret_cast<const WT*>(a.d.rows) + e);
  if constexpr (FTRL) st.z = load_raw<float, EPL>(a.d.linear + e);
  return st;
}

// Element-wise Adagrad on one lane's elements: acc += g^2; w -= lr * g / (sqrt(acc) + eps).
// fp16 rows with a master copy update the master and store its fp16 rounding as the row.  The
// square root and the reciprocal are the hardware's (v_sqrt_f32, v_rcp_f32, about 1 ulp each);
// the correctly rounded forms cost ~35 instructions per element, which made them the largest
// share of the update kernel's instructions.  The error they add to the step (a few ulp of the
// step) is far inside the fp32 parity tolerance.
//
// FTRL-Proximal per coordinate (McMahan et al. 2013, Algorithm 1; the sparse-optimizer passage of
// the JD article names FTRL as the Adagrad variant for sparse features), with the accumulator as
// the squared-gradient sum n and w the stored weight:
//   n' = n + g^2,  sigma = (sqrt(n') - sqrt(n)) / alpha,  z' = z + g - sigma * w,
//   w' = 0 if |z'| <= l1, else -(z' - sign(z') l1) / ((beta + sqrt(n')) / alpha + l2).
template <typename RowT, int EPL, bool MASTER, bool FTRL>
__device__ __forceinline__ void apply_state(const UpdArgs& a, uint32_t r, int e0,
                                            typename F32V<EPL>::t g,
                                            const RawState<RowT, EPL, MASTER, FTRL>& st) {
  typedef typename F32V<EPL>::t V;
  typedef typename RawState<RowT, EPL, MASTER, FTRL>::WT WT;
  const uint64_t e = (uint64_t)r * a.d.granule + e0;
  if constexpr (FTRL) {
    const V n0 = to_f32<float, EPL>(st.acc);
    const V n1 = n0 + g * g;
    const V w0 = to_f32<WT, EPL>(st.w);
    V z1 = to_f32<float, EPL>(st.z) + g;
    V w1;
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      const float s1 = __builtin_amdgcn_sqrtf(n1[q]);
      const float sigma = (s1 - __builtin_amdgcn_sqrtf(n0[q])) * a.inv_alpha;
      z1[q] -= sigma * w0[q];
      const float den = (a.beta + s1) * a.inv_alpha + a.l2;
      const float shrunk = z1[q] - __builtin_copysignf(a.l1, z1[q]);
      w1[q] = __builtin_fabsf(z1[q]) <= a.l1 ? 0.0f : -shrunk * __builtin_amdgcn_rcpf(den);
    }
    store_from_f32<float, EPL>(a.d.acc + e, n1);
    store_from_f32<float, EPL>(a.d.linear + e, z1);
    if (MASTER) store_from_f32<float, EPL>(a.d.master + e, w1);
    store_from_f32<RowT, EPL>(reinterpret_cast<RowT*>(a.d.rows) + e, w1);
    return;
  }
  const V acc = to_f32<float, EPL>(st.acc) + g * g;
  V den;
#pragma unroll
  for (int q = 0; q < EPL; ++q) den[q] = __builtin_amdgcn_rcpf(__builtin_amdgcn_sqrtf(acc[q]) + a.eps);
  const V w = to_f32<WT, EPL>(st.w) - (a.lr * g) * den;
  store_from_f32<float, EPL>(a.d.acc + e, acc);
  if (MASTER) store_from_f32<float, EPL>(a.d.master + e, w);
  store_from_f32<RowT, EPL>(reinterpret_cast<RowT*>(a.d.rows) + e, w);
}

// Records that the row at rowref r (D elements wide) was updated: its rowref units' bits in the
// touched bitmap (when the table keeps one).  Called by one lane per row.  A row spans at most
// 32 units (dims are at most 256, granules at least 8), so its bits fall in one or two words.
__device__ __forceinline__ void mark_touched(const DevDesc& d, uint32_t r, int D) {
  if (!d.touched) return;
  const int units = D / d.granule;
  const uint64_t m = ((1ull << units) - 1ull) << (r & 31u);
  atomicOr(d.touched + (r >> 5), (uint32_t)m);
  if ((uint32_t)(m >> 32)) atomicOr(d.touched + (r >> 5) + 1, (uint32_t)(m >> 32));
}

// Issues the load of one occurrence's upstream-gradient slice (bag `bag`, lane elements from e0);
// returns the raw slice, the row width D of the bag's field and whether the lane is in use.
template <typename GradT, int EPL, bool VAR>
__device__ __forceinline__ typename VecOf<GradT, EPL>::t grad_raw(const UpdArgs& a, uint32_t bag,
                                                                  int e0, bool on, int& D,
                                                                  bool& ok) {
  const uint32_t b = div_fields(a.d, bag);
  const int f = (int)(bag - b * (uint32_t)a.d.n_fields);
  D = VAR ? a.d.fdim[f] : a.d.fixed_dim;
  const int col = VAR ? a.d.fcol[f] : f * a.d.fixed_dim;
  ok = on && e0 < D;
  const GradT* G = reinterpret_cast<const GradT*>(a.grad) + e0;
  return load_raw<GradT, EPL>(G + (ok ? (uint64_t)b * a.d.out_width + col : 0ull));
}

template <int EPL> struct SegBatch { static constexpr int value = EPL == 4 ? 4 : 2; };

constexpr uint32_t kHeadEnds = 1u, kHeadPasses = 2u;

constexpr int kPieceMax = 256;  // occurrences per update piece, at most
constexpr int kPieceMin = 192;  // occurrences per update piece, at least (while the batch allows)

// Carries of the segments that cross lane-group boundaries inside a piece, combined once per
// piece: group g contributes (reset, v, valid) where reset means the carry it passes on does not
// include what reached it.  Inclusive segmented scan over the wave's groups (stride GS lanes).
template <int EPL>
__device__ __forceinline__ void group_scan(int gs_log2, int g, bool& reset,
                                           typename F32V<EPL>::t& v, bool& valid) {
  typedef typename F32V<EPL>::t V;
  const int GS = 1 << gs_log2;
  const int IPR = 64 >> gs_log2;
  for (int d = 1; d < IPR; d <<= 1) {
    V y;
#pragma unroll
    for (int q = 0; q < EPL; ++q) y[q] = __shfl_up(v[q], d * GS, 64);
    const int rv = __shfl_up((int)reset | ((int)valid << 1), d * GS, 64);
    if (g >= d && !reset) {
      v += y;
      valid = (rv >> 1) & 1;
      reset = rv & 1;
    }
  }
}

// Segmented gradient reduction in sorted order fused with the Adagrad update.  A wave owns pieces
// of IPR x K consecutive sorted occurrences (IPR = 64 / GS lane groups of GS lanes; `rounds` is
// K); lane group g takes the piece's occurrences g*K .. g*K+K-1 and sums them one after another,
// restarting at each segment head (segments are runs of equal rows).  A segment that begins and
// ends inside one group is applied there, its state loads issued with the gradient loads of the
// batch that ends it.  The segments that cross group boundaries are joined once per piece by a
// segmented scan over the groups; those that end inside the piece are applied by the group where
// they end.  The piece's first segment, when it began in an earlier piece, is left as a head
// partial, and its last segment, when it runs into the next piece, as a tail partial;
// k_update_fixup joins them.  The piece's sorted keys (with one neighbour on each side) and bags
// are staged in the wave's LDS region first, with coalesced loads.
template <typename RowT, typename GradT, bool VAR, bool MASTER, bool TRACK, bool FTRL>
__global__ __launch_bounds__(kBlock, 4) void k_update_pieces(UpdArgs a, int gs_log2) {
  constexpr int EPL = 16 / (int)sizeof(RowT);
  constexpr int BR = SegBatch<EPL>::value;
  constexpr int kStage = (kPieceMax + 2 + 63) / 64;
  typedef typename F32V<EPL>::t V;
  __shared__ uint32_t s_heads;
  __shared__ uint32_t s_key[kWaves][kPieceMax + 2];
  __shared__ uint32_t s_val[kWaves][kPieceMax];
  if (threadIdx.x == 0) s_heads = 0;
  __syncthreads();
  const int PW = a.pw;
  const int lane = lane_id();
  const int wv = threadIdx.x >> 6;
  const uint32_t NONE = 0xFFFFFFFFu;  // above every row key; equal to the miss key
  // rowref part of a sort key (mixed-width tables carry the width class above it)
  const uint32_t rmask = a.d.classed ? (1u << a.d.cls_shift) - 1u : 0xFFFFFFFFu;
  uint32_t* sk = s_key[wv];
  uint32_t* sv = s_val[wv];
  const int64_t wstride = (int64_t)gridDim.x * (kBlock / 64);
  uint32_t heads = 0;
  for (int64_t c = ((int64_t)blockIdx.x * kBlock + threadIdx.x) / 64; c < a.n_pieces; c += wstride) {
    const int64_t p0 = c * PW;
    const int64_t p1 = min((int64_t)a.n, p0 + PW);
    // stage keys[p0-1 .. p0+PW] and bags[p0 .. p0+PW) in LDS (clamped reads, then masking)
    {
      uint32_t kv[kStage], vv[kStage];
#pragma unroll
      for (int q = 0; q < kStage; ++q) {
        const int64_t idx = p0 - 1 + q * 64 + lane;
        kv[q] = a.key[min(max(idx, (int64_t)0), (int64_t)a.n - 1)];
        vv[q] = a.val[min(p0 + q * 64 + lane, (int64_t)a.n - 1)];
      }
#pragma unroll
      for (int q = 0; q < kStage; ++q) {
        const int j = q * 64 + lane;
        const int64_t idx = p0 - 1 + j;
        if (j < PW + 2) sk[j] = (idx >= 0 && idx < a.n) ? kv[q] : NONE;
        if (j < PW) sv[j] = p0 + j < p1 ? vv[q] : 0u;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // touched bitmap: each row is marked by the piece holding its first occurrence (a separate
    // instantiation, so the update of untracked tables carries none of it)
    if (TRACK) {
      for (int j = lane; j < PW; j += 64) {
        const uint32_t kj = sk[j + 1];
        if (kj < a.miss_key && kj != sk[j]) {
          const uint32_t b = div_fields(a.d, sv[j]);
          const int f = (int)(sv[j] - b * (uint32_t)a.d.n_fields);
          mark_touched(a.d, kj & rmask, a.d.var_dim ? a.d.fdim[f] : a.d.fixed_dim);
        }
      }
    }
    // lane groups: as wide as the piece's widest rows (its last key's width class, the classes
    // being sorted above the rowrefs), else the table's widest
    int gsl = gs_log2;
    if (a.d.classed && sk[PW] < a.miss_key) gsl = (int)(sk[PW] >> a.d.cls_shift);
    const int GS = 1 << gsl;
    const int IPR = 64 >> gsl;
    const int K = PW / IPR;
    const int li = lane & (GS - 1);
    const int g = lane >> gsl;
    const int e0 = li * EPL;
    // sk[j + 1] is the key of piece position j
    const int j0 = g * K;
    const uint32_t kfirst = sk[j0 + 1];
    // the group's first segment began before the group
    const bool gcont = kfirst < a.miss_key && sk[j0] == kfirst;
    V s = 0.0f;          // running sum of the current segment
    V hsum = 0.0f;       // the group's first segment, when it began earlier and ends in the group
    bool hends = false;
    int gD = 0;          // row width of the group's first occurrence
    for (int k0 = 0; k0 < K; k0 += BR) {
      uint32_t kk[BR];
      bool hd[BR], upd[BR], hend[BR], okg[BR];
      typename VecOf<GradT, EPL>::t gr[BR];
      RawState<RowT, EPL, MASTER, FTRL> st[BR];
      int D[BR];
      // issue every load of the batch: gradient slices and the state of rows ending here
#pragma unroll
      for (int r = 0; r < BR; ++r) {
        const int j = j0 + k0 + r;
        const uint32_t kr = sk[j + 1];
        const bool own = kr < a.miss_key;
        const bool in_grp = own && !(gcont && kr == kfirst);
        const bool end = own && sk[j + 2] != kr;
        kk[r] = own ? kr : NONE;
        hd[r] = own && sk[j] != kr;
        gr[r] = grad_raw<GradT, EPL, VAR>(a, sv[j], e0, own, D[r], okg[r]);
        upd[r] = end && in_grp && okg[r];
        hend[r] = end && !in_grp;
        st[r] = load_state<RowT, EPL, MASTER, FTRL>(a, kk[r] & rmask, e0, upd[r]);
      }
      if (k0 == 0) gD = D[0];
#pragma unroll
      for (int r = 0; r < BR; ++r) {
        const V x = okg[r] ? to_f32<GradT, EPL>(gr[r]) : V(0.0f);
        s = hd[r] ? x : s + x;
        heads += (hd[r] && li == 0) ? 1u : 0u;
        if (upd[r]) apply_state<RowT, EPL, MASTER, FTRL>(a, kk[r] & rmask, e0, s, st[r]);
        if (hend[r]) {
          hsum = s;
          hends = true;
        }
      }
    }
    // what this group passes on: its last segment when that runs past the group's end
    const uint32_t klast = sk[j0 + K];
    const bool lown = klast < a.miss_key;
    const bool lcont = lown && sk[j0 + K + 1] == klast;       // runs past the group's end
    const bool passes = gcont && !hends && lown && klast == kfirst && lcont;
    const bool tf = lcont && !passes;                          // began inside the group
    // group scan: reset unless the group passes its carry through; the carry is then the
    // group's sum (its whole range) added to what reached it, else its tail sum
    bool reset = !passes;
    V v = (passes || tf) ? s : V(0.0f);
    bool valid = tf;
    group_scan<EPL>(gsl, g, reset, v, valid);
    // carry reaching group g: the inclusive value of group g - 1; group 0 receives the piece's
    // head chain (nothing summed yet here, valid when the piece begins inside a segment)
    const bool cont = sk[1] < a.miss_key && sk[0] == sk[1];
    V cin;
#pragma unroll
    for (int q = 0; q < EPL; ++q) cin[q] = __shfl_up(v[q], GS, 64);
    const int rvin = __shfl_up((int)reset | ((int)valid << 1), GS, 64);
    if (g == 0) cin = 0.0f;
    // head partial ending in this group: the piece's first segment (begun in an earlier piece,
    // passed through every group before this one) or a row begun in an earlier group
    uint32_t flag = 0;
    const bool chain_ends = gcont && hends;
    const bool piece_head_ends = chain_ends && cont && (g == 0 || !(rvin & 1));
    const bool row_ends = chain_ends && !piece_head_ends;
    const V total = cin + hsum;
    const RawState<RowT, EPL, MASTER, FTRL> sth =
        load_state<RowT, EPL, MASTER, FTRL>(a, kfirst & rmask, e0, row_ends && e0 < gD);
    if (row_ends && e0 < gD) apply_state<RowT, EPL, MASTER, FTRL>(a, kfirst & rmask, e0, total, sth);
    if (piece_head_ends && e0 < gD) store_from_f32<float, EPL>(a.phead + c * a.pdim + e0, total);
    if (__ballot(piece_head_ends) != 0) flag |= kHeadEnds << 1;
    // the last group's carry runs into the next piece
    const int src = (IPR - 1) * GS + li;
    V cl;
#pragma unroll
    for (int q = 0; q < EPL; ++q) cl[q] = __shfl(v[q], src, 64);
    const int rvl = __shfl((int)reset | ((int)valid << 1), src, 64);
    const uint32_t kl = __shfl(klast, src, 64);
    // valid at the last group: its tail, or a pass-through chain that began at a tail (valid) or
    // at the piece's head (no reset anywhere and the piece began inside a segment)
    const bool l_reset = rvl & 1, l_valid = (rvl >> 1) & 1;
    const bool whole_piece = !l_reset && cont;  // one segment across the whole piece
    if (whole_piece) {
      flag |= kHeadPasses << 1;
      if (g == 0 && e0 < gD) store_from_f32<float, EPL>(a.phead + c * a.pdim + e0, cl);
    } else if (l_valid) {
      flag |= 1u;
      // row width of the tail's row: that of the last group's last occurrence
      int Dl;
      bool okl;
      const uint32_t bag_l = sv[min((IPR - 1) * K + K - 1, PW - 1)];
      (void)grad_raw<GradT, EPL, VAR>(a, bag_l, e0, false, Dl, okl);
      if (g == 0 && e0 < Dl) store_from_f32<float, EPL>(a.ptail + c * a.pdim + e0, cl);
      if (lane == 0) {
        a.pkey[2 * c] = kl & rmask;
        a.pkey[2 * c + 1] = (uint32_t)Dl;
      }
    }
    if (lane == 0) a.pflag[c] = flag;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
  }
  // heads were counted by the first lane of each group, whatever the group width per piece
  uint32_t wsum = heads;
  for (int d = 32; d >= 1; d >>= 1) wsum += __shfl_xor(wsum, d, 64);
  if (lane == 0 && wsum) atomicAdd(&s_heads, wsum);
  __syncthreads();
  if (threadIdx.x == 0 && s_heads) atomicAdd(&a.ctr[1], s_heads);
}

// Joins the partial sums of segments that cross pieces.  One wave per piece with a tail partial:
// it reads the flags of the following pieces 64 at a time to find where the segment ends, adds the
// head partials of those pieces in order (lane groups take alternate pieces, then a wave
// reduction), and applies the update to the row.
template <typename RowT, bool MASTER, bool FTRL>
__global__ __launch_bounds__(kBlock) void k_update_fixup(UpdArgs a, int gs_log2) {
  constexpr int EPL = 16 / (int)sizeof(RowT);
  typedef typename F32V<EPL>::t V;
  const int GS = 1 << gs_log2;
  const int IPR = 64 >> gs_log2;
  const int lane = lane_id();
  const int li = lane & (GS - 1);
  const int g = lane >> gs_log2;
  const int e0 = li * EPL;
  const int64_t wstride = (int64_t)gridDim.x * (kBlock / 64);
  if (blockIdx.x == 0 && threadIdx.x == 0 && a.n_unique) *a.n_unique = (int64_t)a.ctr[1];
  for (int64_t t = ((int64_t)blockIdx.x * kBlock + threadIdx.x) / 64; t < a.n_pieces; t += wstride) {
    if (!(a.pflag[t] & 1u)) continue;
    const uint32_t k = a.pkey[2 * t];
    const int D = (int)a.pkey[2 * t + 1];
    const bool on = e0 < D;
    const bool lead = g == 0 && on;
    const RawState<RowT, EPL, MASTER, FTRL> st = load_state<RowT, EPL, MASTER, FTRL>(a, k, e0, lead);
    const typename VecOf<float, EPL>::t tail =
        load_raw<float, EPL>(a.ptail + (lead ? t * a.pdim : 0) + e0);
    V sum = lead ? to_f32<float, EPL>(tail) : V(0.0f);
    for (int64_t u0 = t + 1; u0 < a.n_pieces; u0 += 64) {
      // pieces u0 .. u0+63: the chain runs through PASS pieces up to the first END piece
      const int64_t u = u0 + lane;
      const uint32_t hk = u < a.n_pieces ? (a.pflag[u] >> 1) & 3u : 0u;
      const uint64_t stop = __ballot(hk != kHeadPasses);
      const int last = stop ? __builtin_ctzll(stop) : 63;  // index of the ending piece
      for (int q0 = 0; q0 <= last; q0 += 4 * IPR) {
        typename VecOf<float, EPL>::t h[4];
        bool use[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int q = q0 + v * IPR + g;
          use[v] = on && q <= last && u0 + q < a.n_pieces;
          h[v] = load_raw<float, EPL>(a.phead + (use[v] ? (u0 + q) * a.pdim : 0) + e0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) sum += use[v] ? to_f32<float, EPL>(h[v]) : V(0.0f);
      }
      if (stop) break;
    }
    // reduce the groups' sums into group 0
    for (int d = IPR >> 1; d >= 1; d >>= 1) {
#pragma unroll
      for (int q = 0; q < EPL; ++q) sum[q] += __shfl_down(sum[q], d * GS, 64);
    }
    if (lead) apply_state<RowT, EPL, MASTER, FTRL>(a, k, e0, sum, st);
  }
}

// ---------------------------------------------------------------- optional unique list output
struct SegArgs {
  const uint32_t* key;
  int32_t n;
  int32_t tiles;
  int32_t tile;       // items per tile
  uint32_t miss_key;
  uint32_t* seg;      // [tiles + 1] head counts -> exclusive offsets; [tiles] = U
  uint32_t* headpos;  // [n + 1] position of each head
  uint32_t* unique;
  int32_t* count;
  uint32_t* nvalid;   // one word: number of non-miss occurrences
  uint32_t rmask;     // rowref part of a sort key
};

__device__ __forceinline__ bool seg_head(const SegArgs& a, int32_t i) {
  const uint32_t k = a.key[i];
  return k != a.miss_key && (i == 0 || a.key[i - 1] != k);
}

__global__ __launch_bounds__(kBlock) void k_seg_count(SegArgs a) {
  __shared__ uint32_t s_c, s_v;
  if (threadIdx.x == 0) { s_c = 0; s_v = 0; }
  __syncthreads();
  const int32_t i0 = blockIdx.x * a.tile, i1 = min(a.n, i0 + a.tile);
  uint32_t c = 0, v = 0;
  for (int32_t i = i0 + threadIdx.x; i < i1; i += kBlock) {
    c += seg_head(a, i);
    v += a.key[i] != a.miss_key;
  }
  if (c) atomicAdd(&s_c, c);
  if (v) atomicAdd(&s_v, v);
  __syncthreads();
  if (threadIdx.x == 0) {
    a.seg[blockIdx.x] = s_c;
    if (s_v) atomicAdd(a.nvalid, s_v);
  }
}

__global__ __launch_bounds__(kBlock) void k_seg_scan(SegArgs a) {
  __shared__ uint32_t s_w[kWaves];
  uint32_t carry = 0;
  for (int32_t c0 = 0; c0 < a.tiles; c0 += kBlock) {
    const int32_t i = c0 + threadIdx.x;
    const uint32_t v = i < a.tiles ? a.seg[i] : 0u;
    uint32_t total;
    const uint32_t pre = block_excl_scan(v, s_w, total);
    if (i < a.tiles) a.seg[i] = pre + carry;
    carry += total;
  }
  if (threadIdx.x == 0) a.seg[a.tiles] = carry;
}

__global__ __launch_bounds__(kBlock) void k_seg_write(SegArgs a) {
  __shared__ uint32_t s_w[kWaves];
  const int32_t i0 = blockIdx.x * a.tile;
  uint32_t base = a.seg[blockIdx.x];
  for (int32_t c = 0; c < a.tile; c += kBlock) {
    const int32_t i = i0 + c + threadIdx.x;
    const bool h = (i < a.n) && seg_head(a, i);
    uint32_t total;
    const uint32_t pre = block_excl_scan(h ? 1u : 0u, s_w, total);
    if (h) {
      a.unique[base + pre] = a.key[i] & a.rmask;
      a.headpos[base + pre] = (uint32_t)i;
    }
    base += total;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) a.headpos[a.seg[a.tiles]] = *a.nvalid;
}

__global__ __launch_bounds__(kBlock) void k_seg_counts(SegArgs a) {
  const uint32_t U = a.seg[a.tiles];
  for (uint32_t u = blockIdx.x * kBlock + threadIdx.x; u < U; u += gridDim.x * kBlock)
    a.count[u] = (int32_t)(a.headpos[u + 1] - a.headpos[u]);
}

__global__ void k_zero_words(uint32_t* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0;
}
__global__ void k_set_i64(int64_t* p, int64_t v) { *p = v; }

int log2_group(int dmax, int epl) {
  int lanes = (dmax + epl - 1) / epl, g = 0;
  while ((1 << g) < lanes) ++g;
  return g;
}

}  // namespace

// ---------------------------------------------------------------- layout build on the device
static_assert(kBuildTile == kBlock * kBuildIpt, "build tile");
__device__ __forceinline__ int64_t shfl_up_i64(int64_t v, int d) {
  const int lo = __shfl_up((int)(uint32_t)(uint64_t)v, d, 64);
  const int hi = __shfl_up((int)((uint64_t)v >> 32), d, 64);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
}
__device__ __forceinline__ int64_t shfl_xor_i64(int64_t v, int d) {
  const int lo = __shfl_xor((int)(uint32_t)(uint64_t)v, d, 64);
  const int hi = __shfl_xor((int)((uint64_t)v >> 32), d, 64);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
}
// Exclusive block-wide (max, sum) scan of one (m, u) pair per thread; totals returned by reference.
__device__ __forceinline__ void block_excl_maxsum(int64_t m, uint32_t u, int64_t& m_pre, uint32_t& u_pre,
                                                  int64_t& m_tot, uint32_t& u_tot, int64_t* s_m,
                                                  uint32_t* s_u) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
  int64_t mi = m;
  uint32_t ui = u;
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t om = shfl_up_i64(mi, d);
    const uint32_t ou = __shfl_up(ui, d, 64);
    if (lane >= d) {
      mi = om > mi ? om : mi;
      ui += ou;
    }
  }
  if (lane == 63) {
    s_m[w] = mi;
    s_u[w] = ui;
  }
  __syncthreads();
  int64_t wm = INT64_MIN, tm = INT64_MIN;
  uint32_t wu = 0, tu = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int64_t x = s_m[i];
    const uint32_t y = s_u[i];
    if (i < w) {
      wm = x > wm ? x : wm;
      wu += y;
    }
    tm = x > tm ? x : tm;
    tu += y;
  }
  __syncthreads();
  int64_t pm = shfl_up_i64(mi, 1);
  uint32_t pu = __shfl_up(ui, 1, 64);
  if (lane == 0) {
    pm = INT64_MIN;
    pu = 0;
  }
  m_pre = pm > wm ? pm : wm;
  u_pre = pu + wu;
  m_tot = tm;
  u_tot = tu;
}

__global__ __launch_bounds__(kBlock) void k_build_homes(BuildArgs a) {
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < a.n;
       i += (int64_t)gridDim.x * kBlock) {
    const uint64_t k = a.keys[i];
    const bool t1 = a.n_tables == 2 && (k & 1ull);
    const uint32_t h = home_slot(mix64(k), t1 ? a.n_home1 : a.n_home0);
    a.skey[i] = t1 ? a.n_home0 + h : h;
    a.sval[i] = (uint32_t)i;
  }
}

// Runs of equal sort keys (one home) are short; the thread at each run's start orders the run by
// key (insertion sort) and flags equal keys.
__global__ __launch_bounds__(kBlock) void k_build_ties(BuildArgs a) {
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < a.n;
       i += (int64_t)gridDim.x * kBlock) {
    const uint32_t h = a.sk[i];
    if (i > 0 && a.sk[i - 1] == h) continue;
    int64_t j = i + 1;
    while (j < a.n && a.sk[j] == h) ++j;
    if (j - i < 2) continue;
    for (int64_t p = i + 1; p < j; ++p) {
      const uint32_t v = a.sv[p];
      const uint64_t k = a.keys[v];
      int64_t q = p - 1;
      while (q >= i && a.keys[a.sv[q]] > k) {
        a.sv[q + 1] = a.sv[q];
        --q;
      }
      a.sv[q + 1] = v;
    }
    for (int64_t p = i + 1; p < j; ++p)
      if (a.keys[a.sv[p]] == a.keys[a.sv[p - 1]]) atomicOr(a.dup, 1u);
  }
}

__device__ __forceinline__ uint32_t build_units(const BuildArgs& a, int64_t i) {
  return (uint32_t)a.gran[(int)(a.keys[a.sv[i]] >> 48)];
}

// Per block of kBlock x kBuildIpt items of the segment: max of (home - local index), row units.
__global__ __launch_bounds__(kBlock) void k_build_blocks(BuildArgs a) {
  __shared__ int64_t s_m[kWaves];
  __shared__ uint32_t s_u[kWaves];
  const int64_t i0 = a.s0 + ((int64_t)blockIdx.x * kBlock + threadIdx.x) * kBuildIpt;
  int64_t m = INT64_MIN;
  uint32_t u = 0;
#pragma unroll
  for (int q = 0; q < kBuildIpt; ++q) {
    const int64_t i = i0 + q;
    if (i < a.s1) {
      const int64_t v = (int64_t)(a.sk[i] - a.home_base) - (i - a.s0);
      m = v > m ? v : m;
      u += build_units(a, i);
    }
  }
  int64_t mp, mt;
  uint32_t up, ut;
  block_excl_maxsum(m, u, mp, up, mt, ut, s_m, s_u);
  if (threadIdx.x == 0) {
    a.bmax[blockIdx.x] = mt;
    a.bsum[blockIdx.x] = ut;
  }
}

// One block: exclusive prefix max / sum over the per-block values; totals at [blocks].
__global__ __launch_bounds__(kBlock) void k_build_bscan(BuildArgs a) {
  __shared__ int64_t s_m[kWaves];
  __shared__ uint32_t s_u[kWaves];
  int64_t cm = INT64_MIN;
  uint32_t cu = 0;
  for (int64_t c0 = 0; c0 < a.blocks; c0 += kBlock) {
    const int64_t i = c0 + threadIdx.x;
    const int64_t m = i < a.blocks ? a.bmax[i] : INT64_MIN;
    const uint32_t u = i < a.blocks ? a.bsum[i] : 0u;
    int64_t mp, mt;
    uint32_t up, ut;
    block_excl_maxsum(m, u, mp, up, mt, ut, s_m, s_u);
    if (i < a.blocks) {
      a.bmax[i] = mp > cm ? mp : cm;
      a.bsum[i] = cu + up;
    }
    cm = mt > cm ? mt : cm;
    cu += ut;
  }
  if (threadIdx.x == 0) {
    a.bmax[a.blocks] = cm;
    a.bsum[a.blocks] = cu;
  }
}

// Slots and rowrefs of the segment's items; each key goes to its bucket word, and each item writes
// the prefix word of every bucket from the one after its predecessor's up to its own (the rowref
// of the first key at or after the bucket's start).
__global__ __launch_bounds__(kBlock) void k_build_place(BuildArgs a) {
  __shared__ int64_t s_m[kWaves];
  __shared__ uint32_t s_u[kWaves];
  const int64_t i0 = a.s0 + ((int64_t)blockIdx.x * kBlock + threadIdx.x) * kBuildIpt;
  int64_t v[kBuildIpt];
  uint32_t un[kBuildIpt];
  int64_t m = INT64_MIN;
  uint32_t u = 0;
#pragma unroll
  for (int q = 0; q < kBuildIpt; ++q) {
    const int64_t i = i0 + q;
    v[q] = INT64_MIN;
    un[q] = 0;
    if (i < a.s1) {
      v[q] = (int64_t)(a.sk[i] - a.home_base) - (i - a.s0);
      un[q] = build_units(a, i);
    }
    m = v[q] > m ? v[q] : m;
    u += un[q];
  }
  int64_t mp, mt;
  uint32_t up, ut;
  block_excl_maxsum(m, u, mp, up, mt, ut, s_m, s_u);
  const int64_t cmb = a.bmax[blockIdx.x];
  int64_t run_m = mp > cmb ? mp : cmb;     // max over the segment's items before this one
  uint32_t run_u = a.bsum[blockIdx.x] + up;  // row units before this one
  unsigned long long dsum = 0, dmax = 0;
#pragma unroll
  for (int q = 0; q < kBuildIpt; ++q) {
    const int64_t i = i0 + q;
    if (i >= a.s1) break;
    const int64_t local = i - a.s0;
    const int64_t prev = local > 0 ? (local - 1) + run_m : -1;  // predecessor's slot
    run_m = v[q] > run_m ? v[q] : run_m;
    const uint64_t slot = (uint64_t)(local + run_m);
    const uint32_t rr = a.rowref_base + run_u;
    run_u += un[q];
    const uint64_t b = slot / kKeysPerBucket;
    a.buckets[(a.bucket_base + b) * kWordsPerBucket + (slot - b * kKeysPerBucket)] = a.keys[a.sv[i]];
    const int64_t bp = prev < 0 ? -1 : (int64_t)((uint64_t)prev / kKeysPerBucket);
    for (int64_t c = bp + 1; c <= (int64_t)b; ++c)
      a.buckets[(a.bucket_base + (uint64_t)c) * kWordsPerBucket + 15] = rr;
    const unsigned long long d = (unsigned long long)(run_m - v[q]);
    dsum += d;
    dmax = d > dmax ? d : dmax;
  }
  // displacement statistics: one atomic pair per wave
  for (int o = 32; o >= 1; o >>= 1) {
    dsum += (unsigned long long)shfl_xor_i64((int64_t)dsum, o);
    const unsigned long long x = (unsigned long long)shfl_xor_i64((int64_t)dmax, o);
    dmax = x > dmax ? x : dmax;
  }
  if (lane_id() == 0 && dsum + dmax > 0) {
    atomicAdd(a.disp, dsum);
    atomicMax(a.disp + 1, dmax);
  }
}

__global__ __launch_bounds__(kBlock) void k_build_tail(BuildArgs a) {
  for (uint64_t b = a.tail_from + (uint64_t)blockIdx.x * kBlock + threadIdx.x; b < a.n_buckets;
       b += (uint64_t)gridDim.x * kBlock)
    a.buckets[(a.bucket_base + b) * kWordsPerBucket + 15] = a.tail_value;
}

// ---------------------------------------------------------------- end-of-PASS write-back
__global__ __launch_bounds__(kBlock) void k_wb_count(WbLaunch a) {
  __shared__ uint32_t s_c;
  if (threadIdx.x == 0) s_c = 0;
  __syncthreads();
  const int64_t w0 = (int64_t)blockIdx.x * kWbWords;
  uint32_t c = 0;
  for (int64_t w = w0 + threadIdx.x; w < min(a.n_words, w0 + kWbWords); w += kBlock)
    c += __builtin_popcount(a.touched[w]);
  if (c) atomicAdd(&s_c, c);
  __syncthreads();
  if (threadIdx.x == 0) a.bcount[blockIdx.x] = s_c;
}

__global__ __launch_bounds__(kBlock) void k_wb_scan(WbLaunch a) {
  __shared__ uint32_t s_w[kWaves];
  uint32_t carry = 0;
  for (int64_t c0 = 0; c0 < a.blocks; c0 += kBlock) {
    const int64_t i = c0 + threadIdx.x;
    const uint32_t v = i < a.blocks ? a.bcount[i] : 0u;
    uint32_t total;
    const uint32_t pre = block_excl_scan(v, s_w, total);
    if (i < a.blocks) a.bcount[i] = pre + carry;
    carry += total;
  }
  if (threadIdx.x == 0) a.bcount[a.blocks] = carry;
}

// One block per bitmap block of the range: each thread takes 4 consecutive words, the block scan
// of their bit counts places the set bits, and each set bit's unit (row, accumulator, master and
// FTRL linear elements) is copied to the compact outputs.  The words are cleared once read.
__global__ __launch_bounds__(kBlock) void k_wb_gather(WbLaunch a) {
  __shared__ uint32_t s_w[kWaves];
  const int64_t blk = a.b0 + blockIdx.x;
  const int64_t w0 = blk * kWbWords + (int64_t)threadIdx.x * 4;
  uint32_t bits[4];
  uint32_t c = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    bits[q] = w0 + q < a.n_words ? a.touched[w0 + q] : 0u;
    c += __builtin_popcount(bits[q]);
  }
  uint32_t total;
  uint32_t k = a.bcount[blk] - a.base + block_excl_scan(c, s_w, total);
  const int gb = a.granule * 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t m = bits[q];
    while (m) {
      const int b = __builtin_ctz(m);
      m &= m - 1u;
      const uint64_t unit = (uint64_t)(w0 + q) * 32u + (uint64_t)b;
      a.out_unit[k] = (uint32_t)unit;
      const uint8_t* sr = a.rows + unit * (uint64_t)a.row_bytes;
      uint8_t* dr = a.out_rows + (uint64_t)k * a.row_bytes;
      for (int o = 0; o < a.row_bytes; o += 16)
        *reinterpret_cast<uint4*>(dr + o) = *reinterpret_cast<const uint4*>(sr + o);
      const uint8_t* sa = reinterpret_cast<const uint8_t*>(a.acc + unit * (uint64_t)a.granule);
      uint8_t* da = reinterpret_cast<uint8_t*>(a.out_acc + (uint64_t)k * a.granule);
      for (int o = 0; o < gb; o += 16)
        *reinterpret_cast<uint4*>(da + o) = *reinterpret_cast<const uint4*>(sa + o);
      if (a.has_master) {
        const uint8_t* sm = reinterpret_cast<const uint8_t*>(a.master + unit * (uint64_t)a.granule);
        uint8_t* dm = reinterpret_cast<uint8_t*>(a.out_master + (uint64_t)k * a.granule);
        for (int o = 0; o < gb; o += 16)
          *reinterpret_cast<uint4*>(dm + o) = *reinterpret_cast<const uint4*>(sm + o);
      }
      if (a.linear) {
        const uint8_t* sz = reinterpret_cast<const uint8_t*>(a.linear + unit * (uint64_t)a.granule);
        uint8_t* dz = reinterpret_cast<uint8_t*>(a.out_linear + (uint64_t)k * a.granule);
        for (int o = 0; o < gb; o += 16)
          *reinterpret_cast<uint4*>(dz + o) = *reinterpret_cast<const uint4*>(sz + o);
      }
      ++k;
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (w0 + q < a.n_words && bits[q]) a.touched[w0 + q] = 0u;
}

// ---------------------------------------------------------------- probe statistics
// Sums the forward's partial probe statistics into the caller's counters and clears the slots
// for the next counting launch.  One block.
__global__ __launch_bounds__(kBlock) void k_stats_finish(unsigned long long* pstat,
                                                         unsigned long long* out) {
  __shared__ unsigned long long s[4][kBlock];
  unsigned long long v0 = 0, v1 = 0, v2 = 0, v3 = 0;
  for (int i = threadIdx.x; i < kStatSlots; i += kBlock) {
    unsigned long long* p = pstat + 4 * (size_t)i;
    v0 += p[0];
    v1 += p[1];
    v2 += p[2];
    v3 = p[3] > v3 ? p[3] : v3;
    p[0] = 0;
    p[1] = 0;
    p[2] = 0;
    p[3] = 0;
  }
  s[0][threadIdx.x] = v0;
  s[1][threadIdx.x] = v1;
  s[2][threadIdx.x] = v2;
  s[3][threadIdx.x] = v3;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int t = 1; t < kBlock; ++t) {
      v0 += s[0][t];
      v1 += s[1][t];
      v2 += s[2][t];
      v3 = s[3][t] > v3 ? s[3][t] : v3;
    }
    atomicAdd(out + 0, v0);
    atomicAdd(out + 1, v1);
    atomicAdd(out + 2, v2);
    atomicMax(out + 3, v3);
  }
}

// ---------------------------------------------------------------- batch validation
// One thread per bag: its offsets must not decrease, the first must be 0 and the last nnz; with
// rowrefs, every occurrence of a well-formed bag must be a miss or start a whole row of the bag's
// field inside the table (rowref + the field's row units <= rowref space).
__global__ __launch_bounds__(kBlock) void k_validate(ValArgs a) {
  uint32_t bad = 0;
  for (int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x; j < a.n_bags;
       j += (int64_t)gridDim.x * kBlock) {
    const int32_t o0 = a.offsets[j], o1 = a.offsets[j + 1];
    if (j == 0 && o0 != 0) bad |= 1u;
    if (o1 < o0) bad |= 2u;
    if (j == a.n_bags - 1 && o1 != a.nnz) bad |= 4u;
    if (a.rowref && o0 >= 0 && o1 >= o0 && o1 <= a.nnz) {
      const int f = (int)(j % a.d.n_fields);
      const uint64_t units = (uint64_t)a.d.fgran[f];
      for (int32_t i = o0; i < o1; ++i) {
        const uint32_t r = a.rowref[i];
        if (r != kMiss && (uint64_t)r + units > (uint64_t)a.d.rowref_space) bad |= 8u;
      }
    }
  }
  if (a.n_bags == 0 && a.nnz != 0) bad |= 4u;
  if (bad) atomicOr(a.flag, bad);
}

hipError_t launch_validate(const ValArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(64), 0, st, a.flag, 1);
  if (a.n_bags > 0) {
    const int64_t b = ((int64_t)a.n_bags + kBlock - 1) / kBlock;
    hipLaunchKernelGGL(k_validate, dim3((unsigned)(b < 65536 ? b : 65536)), dim3(kBlock), 0, st, a);
  } else if (a.nnz != 0) {
    hipLaunchKernelGGL(k_validate, dim3(1), dim3(kBlock), 0, st, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- static backward scratch
// The backward's workspace for callers that cannot allocate device memory (code under graph
// capture, allocation-free training loops): one array per device, held until the process ends.
// In host code `scratch` names a host-side stand-in, not the device array; its device address is
// looked up once per device with hipGetSymbolAddress and only that address is used.
constexpr size_t kScratchBytes = 64ull << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

size_t scratch_bytes() { return kScratchBytes; }

hipError_t scratch_address(void** ptr) {
  static std::mutex mu;
  static std::vector<void*> per_device;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if ((size_t)dev >= per_device.size()) per_device.resize((size_t)dev + 1, nullptr);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

// ================================================================ launchers
KTimer::KTimer(LaunchCtx& ctx, const char* name) : c(ctx) {
  if (!c.timing || !c.timing->on) return;
  Timing& T = *c.timing;
  if (!T.only.empty() && T.only != name) return;
  if (T.used == T.pool.size()) {
    Timing::Rec rec{name, nullptr, nullptr};
    if (hipEventCreate(&rec.a) != hipSuccess || hipEventCreate(&rec.b) != hipSuccess) return;
    T.pool.push_back(rec);
  }
  r = &T.pool[T.used++];
  r->name = name;
}

hipError_t launch_lookup_pool(const FwdLaunch& a, LaunchCtx& ctx) {
  if (a.n_bags <= 0) return hipSuccess;
  const int gs = log2_group(a.d.max_dim, a.d.row_f16 ? 8 : 4);
  const dim3 grid((a.n_bags + kFwdBags - 1) / kFwdBags);
  KTimer tm(ctx, a.mode == 1 ? "lookup_probe" : a.mode == 2 ? "pool" : "lookup_pool");
  const dim3 blk(kBlock);
  // the probe form follows the size of the probed bucket array (see the two forms above)
  const uint64_t bucket_bytes =
      ((uint64_t)a.d.tab[0].n_buckets + (a.d.n_tables == 2 ? (uint64_t)a.d.tab[1].n_buckets : 0u)) *
      kWordsPerBucket * 8u;
  const bool coop = a.mode != 2 && (a.probe == 1 || (a.probe == 0 && bucket_bytes >= kCoopProbeBytes));
#define EMB_FWD2(R, O, V, C)                                                                      \
  do {                                                                                            \
    if (a.stats) EMB_LAUNCH(tm, (k_lookup_pool<R, O, V, C, true>), grid, blk, 0, ctx.stream, a, gs); \
    else EMB_LAUNCH(tm, (k_lookup_pool<R, O, V, C, false>), grid, blk, 0, ctx.stream, a, gs);        \
  } while (0)
#define EMB_FWD(R, O, V) do { if (coop) EMB_FWD2(R, O, V, true); else EMB_FWD2(R, O, V, false); } while (0)
  if (a.d.row_f16) {
    if (a.out_f16) { if (a.d.var_dim) EMB_FWD(_Float16, _Float16, true); else EMB_FWD(_Float16, _Float16, false); }
    else { if (a.d.var_dim) EMB_FWD(_Float16, float, true); else EMB_FWD(_Float16, float, false); }
  } else {
    if (a.out_f16) { if (a.d.var_dim) EMB_FWD(float, _Float16, true); else EMB_FWD(float, _Float16, false); }
    else { if (a.d.var_dim) EMB_FWD(float, float, true); else EMB_FWD(float, float, false); }
  }
#undef EMB_FWD
#undef EMB_FWD2
  if (a.stats) {
    KTimer ts(ctx, "probe_stats");
    EMB_LAUNCH(ts, k_stats_finish, dim3(1), blk, 0, ctx.stream, a.d.pstat, a.stats);
  }
  return hipGetLastError();
}

BwdPlan plan_bwd(int64_t nnz, uint32_t rowref_space, int32_t max_dim, int32_t row_f16,
                 int32_t classed) {
  BwdPlan p{};
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.n = (int32_t)nnz;
  // key bits of the largest rowref; fewest passes of at most 8 or 9 bits
  int keybits = 0;
  while (keybits < 32 && rowref_space > 1 && ((uint64_t)(rowref_space - 1) >> keybits) != 0) ++keybits;
  if (classed) keybits += 3;  // the width class above the rowref bits
  // digit width: each tile's per-bin work (count, scan, offsets) must stay small next to its
  // per-item work, and each digit's run of a tile must stay long enough to write in whole lines.
  // Measured on MI355X with 4096-item tiles: 9-bit digits cost no more per pass than 8-bit ones,
  // while 10-bit digits make a pass ~1.9x slower (a 30-bit key sorts faster in 4 passes of 8 bits
  // than in 3 of 10).
  const int maxbits = nnz >= (4 << 20) ? 9 : 8;
  p.passes = keybits <= maxbits ? 1 : (keybits + maxbits - 1) / maxbits;
  p.bits = (keybits + p.passes - 1) / p.passes;
  // tiles: enough of them to spread a small batch over every CU, large ones for large batches
  p.ipt = nnz >= (1 << 20) ? 8 : 4;
  const int64_t tile = (int64_t)kBlock * p.ipt;
  p.tiles = (int32_t)((nnz + tile - 1) / tile);
  const size_t n = (size_t)(nnz > 0 ? nnz : 0);
  const size_t bins = ((size_t)1 << p.bits) + 1;
  size_t o = 0;
  p.off_ka = o; o = al(o + 4 * (n + 1));
  p.off_va = o; o = al(o + 4 * (n + 1));
  p.off_kb = o; o = al(o + 4 * (n + 1));
  p.off_vb = o; o = al(o + 4 * (n + 1));
  p.off_counts = o; o = al(o + 4 * bins * (size_t)(p.tiles > 0 ? p.tiles : 1));
  // tiles per histogram block: keep at least ~512 blocks, at most 16 tiles each
  p.tile_group = p.tiles >= 512 * 16 ? 16 : p.tiles >= 512 ? p.tiles / 512 : 1;
  p.groups = (p.tiles + p.tile_group - 1) / p.tile_group;
  p.off_gsum = o; o = al(o + 4 * bins * (size_t)(p.groups > 0 ? p.groups : 1));
  p.off_tot = o; o = al(o + 4 * bins);
  p.off_ctr = o; o = al(o + 4 * 16);
  p.off_seg = o; o = al(o + 4 * ((size_t)p.tiles + 1));
  // update pieces: about 128k of them (bounded partial traffic), and at least kPieceMin
  // occurrences each.  On the 26-field batch (325k occurrences) pieces of 64, 128, 192 and 256
  // took the update 26.3, 21.8, 21.0 and 23.4 us on MI355X: small pieces cost more in per-piece
  // staging and scans than they gain in spread, very large ones leave too few waves.
  const int epl = row_f16 ? 8 : 4;
  p.gsl = log2_group(max_dim, epl);
  const int ipr = 64 >> p.gsl;
  const int br = row_f16 ? SegBatch<8>::value : SegBatch<4>::value;
  int64_t r = (nnz + (int64_t)ipr * 131072 - 1) / ((int64_t)ipr * 131072);
  const int64_t rmax = kPieceMax / ipr;
  const int64_t rmin = (kPieceMin + ipr - 1) / ipr;
  r = r < rmin ? rmin : r;
  r = r < br ? br : r > rmax ? rmax : r;
  p.rounds = (int32_t)((r + br - 1) / br * br);
  // mixed-width tables: full pieces, each split among as many lane groups as its rows' width allows
  if (classed) p.rounds = (int32_t)rmax;
  const int64_t pw = (int64_t)p.rounds * ipr;
  p.pw = (int32_t)pw;
  p.n_pieces = (int32_t)((nnz + pw - 1) / pw);
  p.pdim = max_dim;
  const size_t np = (size_t)(p.n_pieces > 0 ? p.n_pieces : 1);
  p.off_phead = o; o = al(o + 4 * np * (size_t)p.pdim);
  p.off_ptail = o; o = al(o + 4 * np * (size_t)p.pdim);
  p.off_pflag = o; o = al(o + 4 * np);
  p.off_pkey = o; o = al(o + 8 * np);
  p.bytes = o;
  return p;
}

template <bool FIRST, int IPT>
static void launch_scatter_ipt(const SortArgs& s, int logb, dim3 grid, hipStream_t st, KTimer& tm) {
  const dim3 blk(kBlock);
  switch (logb) {
    case 8: EMB_LAUNCH(tm, (k_sort_scatter<FIRST, IPT, 8>), grid, blk, 0, st, s); break;
    default: EMB_LAUNCH(tm, (k_sort_scatter<FIRST, IPT, 9>), grid, blk, 0, st, s); break;
  }
}

template <bool FIRST>
static void launch_scatter(const SortArgs& s, int ipt, int logb, dim3 grid, hipStream_t st, KTimer& tm) {
  if (ipt == 4) launch_scatter_ipt<FIRST, 4>(s, logb, grid, st, tm);
  else launch_scatter_ipt<FIRST, 8>(s, logb, grid, st, tm);
}

// One launch of the update kernel for the table's row, gradient and state types; tracking and the
// optimizer pick the instantiation.
template <typename R, typename G, bool V, bool M>
void launch_pieces(const UpdArgs& u, int gsl, bool track, bool ftrl, dim3 grid, hipStream_t st,
                   KTimer& tm) {
  const dim3 blk(kBlock);
  if (ftrl) {
    if (track) EMB_LAUNCH(tm, (k_update_pieces<R, G, V, M, true, true>), grid, blk, 0, st, u, gsl);
    else EMB_LAUNCH(tm, (k_update_pieces<R, G, V, M, false, true>), grid, blk, 0, st, u, gsl);
  } else {
    if (track) EMB_LAUNCH(tm, (k_update_pieces<R, G, V, M, true, false>), grid, blk, 0, st, u, gsl);
    else EMB_LAUNCH(tm, (k_update_pieces<R, G, V, M, false, false>), grid, blk, 0, st, u, gsl);
  }
}

hipError_t launch_sparse_bwd(const BwdLaunch& a, const BwdPlan& p, LaunchCtx& ctx) {
  uint8_t* ws = reinterpret_cast<uint8_t*>(a.ws);
  uint32_t* ctr = reinterpret_cast<uint32_t*>(ws + p.off_ctr);
  if (p.n <= 0) {
    if (a.n_unique && a.stage != 1) {
      KTimer tm(ctx, "set_n_unique");
      EMB_LAUNCH(tm, k_set_i64, dim3(1), dim3(1), 0, ctx.stream, a.n_unique, (int64_t)0);
    }
    return hipGetLastError();
  }
  SortArgs s{};
  s.rowref = a.rowref;
  s.offsets = a.offsets;
  s.n_bags = a.n_bags;
  s.counts = reinterpret_cast<uint32_t*>(ws + p.off_counts);
  s.gsum = reinterpret_cast<uint32_t*>(ws + p.off_gsum);
  s.groups = p.groups;
  s.tile_group = p.tile_group;
  s.tot = reinterpret_cast<uint32_t*>(ws + p.off_tot);
  s.ctr = ctr;
  s.n = p.n;
  s.tiles = p.tiles;
  s.tile = kBlock * p.ipt;
  s.rowref_space = a.d.rowref_space;
  s.classed = a.d.classed;
  s.cls_shift = a.d.cls_shift;
  s.fgsl = a.d.fgsl;
  s.n_fields = a.d.n_fields;
  s.fdiv_m = a.d.fdiv_m;
  s.fdiv_s = a.d.fdiv_s;
  s.bits = p.bits;
  const int logb = p.bits <= 8 ? 8 : p.bits;
  uint32_t* ka = reinterpret_cast<uint32_t*>(ws + p.off_ka);
  uint32_t* va = reinterpret_cast<uint32_t*>(ws + p.off_va);
  uint32_t* kb = reinterpret_cast<uint32_t*>(ws + p.off_kb);
  uint32_t* vb = reinterpret_cast<uint32_t*>(ws + p.off_vb);
  const dim3 tiles(p.tiles), blk(kBlock);
  const dim3 nbins((1u << p.bits) + 1);
  uint32_t *src_k = nullptr, *src_v = nullptr, *dst_k = ka, *dst_v = va;
  if (a.stage == 2) {
    // the sort ran in an earlier call: its output is where the last of its passes wrote
    src_k = (p.passes & 1) ? ka : kb;
    src_v = (p.passes & 1) ? va : vb;
    dst_k = (p.passes & 1) ? kb : ka;
    dst_v = (p.passes & 1) ? vb : va;
  }
  for (int pass = 0; pass < p.passes && a.stage != 2; ++pass) {
    s.shift = p.bits * pass;
    s.kin = src_k;
    s.vin = src_v;
    s.kout = dst_k;
    s.vout = dst_v;
    {
      KTimer tm(ctx, "sort_hist");
      if (pass == 0) EMB_LAUNCH(tm, k_sort_hist<true>, dim3(p.groups), blk, 0, ctx.stream, s);
      else EMB_LAUNCH(tm, k_sort_hist<false>, dim3(p.groups), blk, 0, ctx.stream, s);
    }
    {
      KTimer tm(ctx, "sort_scan");
      EMB_LAUNCH(tm, k_sort_scan, nbins, blk, 0, ctx.stream, s, pass == 0 ? 1 : 0);
    }
    {
      KTimer tm(ctx, "sort_scatter");
      if (pass == 0) launch_scatter<true>(s, p.ipt, logb, tiles, ctx.stream, tm);
      else launch_scatter<false>(s, p.ipt, logb, tiles, ctx.stream, tm);
    }
    src_k = dst_k;
    src_v = dst_v;
    dst_k = (src_k == ka) ? kb : ka;
    dst_v = (src_v == va) ? vb : va;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.stage == 1) return err;

  UpdArgs u{};
  u.d = a.d;
  u.key = src_k;
  u.val = src_v;
  u.n = p.n;
  u.miss_key = kMissKey;
  u.grad = a.grad;
  u.lr = a.lr;
  u.eps = a.eps;
  u.inv_alpha = a.ftrl ? 1.0f / a.lr : 0.0f;
  u.beta = a.beta;
  u.l1 = a.l1;
  u.l2 = a.l2;
  u.ctr = ctr;
  u.n_unique = a.n_unique;
  u.rounds = p.rounds;
  u.pw = p.pw;
  u.n_pieces = p.n_pieces;
  u.pdim = p.pdim;
  u.phead = reinterpret_cast<float*>(ws + p.off_phead);
  u.ptail = reinterpret_cast<float*>(ws + p.off_ptail);
  u.pflag = reinterpret_cast<uint32_t*>(ws + p.off_pflag);
  u.pkey = reinterpret_cast<uint32_t*>(ws + p.off_pkey);
  const int gsl = p.gsl;
  const int64_t blocks = ((int64_t)p.n_pieces + (kBlock / 64) - 1) / (kBlock / 64);
  const dim3 gpiece((unsigned)(blocks < 8192 ? blocks : 8192));
  {
    KTimer tm(ctx, "update_pieces");
    const bool var = a.d.var_dim != 0, mst = a.d.has_master != 0;
    const bool track = a.d.touched != nullptr, ftrl = a.ftrl != 0;
    if (a.d.row_f16) {
      if (a.grad_f16) {
        if (var) { if (mst) launch_pieces<_Float16, _Float16, true, true>(u, gsl, track, ftrl, gpiece, ctx.stream, tm);
                   else launch_pieces<_Float16, _Float16, true, false>(u, gsl, track, ftrl, gpiece, ctx.stream, tm); }
        else { if (mst) launch_pieces<_Float16, _Float16, false, true>(u, gsl, track, ftrl, gpiece, ctx.stream, tm);
               else launch_pieces<_Float16, _Float16, false, false>(u, gsl, track, ftrl, gpiece, ctx.stream, tm); }
      } else {
        if (var) { if (mst) launch_pieces<_Float16, float, true, true>(u, gsl, track, ftrl, gpiece, ctx.stream, tm);
                   else launch_pieces<_Float16, float, true, false>(u, gsl, track, ftrl, gpiece, ctx.stream, tm); }
        else { if (mst) launch_pieces<_Float16, float, false, true>(u, gsl, track, ftrl, gpiece, ctx.stream, tm);
               else launch_pieces<_Float16, float, false, false>(u, gsl, track, ftrl, gpiece, ctx.stream, tm); }
      }
    } else {
      if (a.grad_f16) { if (var) launch_pieces<float, _Float16, true, false>(u, gsl, track, ftrl, gpiece, ctx.stream, tm);
                        else launch_pieces<float, _Float16, false, false>(u, gsl, track, ftrl, gpiece, ctx.stream, tm); }
      else { if (var) launch_pieces<float, float, true, false>(u, gsl, track, ftrl, gpiece, ctx.stream, tm);
             else launch_pieces<float, float, false, false>(u, gsl, track, ftrl, gpiece, ctx.stream, tm); }
    }
  }
  {
    KTimer tm(ctx, "update_fixup");
    const bool ftrl = a.ftrl != 0;
    if (a.d.row_f16) {
      if (a.d.has_master) {
        if (ftrl) EMB_LAUNCH(tm, (k_update_fixup<_Float16, true, true>), gpiece, blk, 0, ctx.stream, u, gsl);
        else EMB_LAUNCH(tm, (k_update_fixup<_Float16, true, false>), gpiece, blk, 0, ctx.stream, u, gsl);
      } else {
        if (ftrl) EMB_LAUNCH(tm, (k_update_fixup<_Float16, false, true>), gpiece, blk, 0, ctx.stream, u, gsl);
        else EMB_LAUNCH(tm, (k_update_fixup<_Float16, false, false>), gpiece, blk, 0, ctx.stream, u, gsl);
      }
    } else {
      if (ftrl) EMB_LAUNCH(tm, (k_update_fixup<float, false, true>), gpiece, blk, 0, ctx.stream, u, gsl);
      else EMB_LAUNCH(tm, (k_update_fixup<float, false, false>), gpiece, blk, 0, ctx.stream, u, gsl);
    }
  }
  err = hipGetLastError();
  if (err != hipSuccess || !a.unique) return err;

  SegArgs g{};
  g.key = src_k;
  g.n = p.n;
  g.tiles = p.tiles;
  g.tile = kBlock * p.ipt;
  g.miss_key = kMissKey;
  g.seg = reinterpret_cast<uint32_t*>(ws + p.off_seg);
  g.headpos = dst_k;  // the spare key buffer (n + 1 words)
  g.unique = a.unique;
  g.count = a.count;
  g.nvalid = ctr + 2;
  g.rmask = a.d.classed ? (1u << a.d.cls_shift) - 1u : 0xFFFFFFFFu;
  {
    KTimer tm(ctx, "seg_zero");
    EMB_LAUNCH(tm, k_zero_words, dim3(1), dim3(64), 0, ctx.stream, ctr + 2, 1);
  }
  {
    KTimer tm(ctx, "seg_count");
    EMB_LAUNCH(tm, k_seg_count, tiles, blk, 0, ctx.stream, g);
  }
  {
    KTimer tm(ctx, "seg_scan");
    EMB_LAUNCH(tm, k_seg_scan, dim3(1), blk, 0, ctx.stream, g);
  }
  {
    KTimer tm(ctx, "seg_write");
    EMB_LAUNCH(tm, k_seg_write, tiles, blk, 0, ctx.stream, g);
  }
  if (a.count) {
    KTimer tm(ctx, "seg_counts");
    EMB_LAUNCH(tm, k_seg_counts, dim3(1024), blk, 0, ctx.stream, g);
  }
  return hipGetLastError();
}

static unsigned grid_for(int64_t n, int64_t cap) {
  const int64_t b = (n + kBlock - 1) / kBlock;
  return (unsigned)(b < 1 ? 1 : b > cap ? cap : b);
}

hipError_t launch_build_homes(const BuildArgs& a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_build_homes, dim3(grid_for(a.n, 65536)), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_build_ties(const BuildArgs& a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_build_ties, dim3(grid_for(a.n, 65536)), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_build_scan(const BuildArgs& a, hipStream_t st) {
  if (a.blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_build_blocks, dim3((unsigned)a.blocks), dim3(kBlock), 0, st, a);
  hipLaunchKernelGGL(k_build_bscan, dim3(1), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_build_place(const BuildArgs& a, hipStream_t st) {
  if (a.blocks > 0)
    hipLaunchKernelGGL(k_build_place, dim3((unsigned)a.blocks), dim3(kBlock), 0, st, a);
  if (a.tail_from < a.n_buckets)
    hipLaunchKernelGGL(k_build_tail, dim3(grid_for((int64_t)(a.n_buckets - a.tail_from), 65536)),
                       dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_build_sort(const BuildArgs& a, const BwdPlan& p, uint8_t* ws, uint32_t** ks,
                             uint32_t** vs, hipStream_t st) {
  SortArgs s{};
  s.counts = reinterpret_cast<uint32_t*>(ws + p.off_counts);
  s.gsum = reinterpret_cast<uint32_t*>(ws + p.off_gsum);
  s.groups = p.groups;
  s.tile_group = p.tile_group;
  s.tot = reinterpret_cast<uint32_t*>(ws + p.off_tot);
  s.ctr = reinterpret_cast<uint32_t*>(ws + p.off_ctr);
  s.n = p.n;
  s.tiles = p.tiles;
  s.tile = kBlock * p.ipt;
  s.rowref_space = 0xFFFFFFFFu;
  s.bits = p.bits;
  const int logb = p.bits <= 8 ? 8 : p.bits;
  uint32_t* ka = reinterpret_cast<uint32_t*>(ws + p.off_ka);
  uint32_t* va = reinterpret_cast<uint32_t*>(ws + p.off_va);
  uint32_t* kb = reinterpret_cast<uint32_t*>(ws + p.off_kb);
  uint32_t* vb = reinterpret_cast<uint32_t*>(ws + p.off_vb);
  uint32_t *src_k = ka, *src_v = va, *dst_k = kb, *dst_v = vb;
  LaunchCtx ctx{st, nullptr};
  KTimer tm(ctx, "build_sort");
  const dim3 tiles(p.tiles), blk(kBlock), nbins((1u << p.bits) + 1);
  for (int pass = 0; pass < p.passes && p.n > 0; ++pass) {
    s.shift = p.bits * pass;
    s.kin = src_k;
    s.vin = src_v;
    s.kout = dst_k;
    s.vout = dst_v;
    hipLaunchKernelGGL(k_sort_hist<false>, dim3(p.groups), blk, 0, st, s);
    hipLaunchKernelGGL(k_sort_scan, nbins, blk, 0, st, s, pass == 0 ? 1 : 0);
    launch_scatter<false>(s, p.ipt, logb, tiles, st, tm);
    std::swap(src_k, dst_k);
    std::swap(src_v, dst_v);
  }
  *ks = src_k;
  *vs = src_v;
  (void)a;
  return hipGetLastError();
}

hipError_t launch_wb_count(const WbLaunch& a, hipStream_t st) {
  if (a.blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_wb_count, dim3((unsigned)a.blocks), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_wb_scan(const WbLaunch& a, hipStream_t st) {
  if (a.blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_wb_scan, dim3(1), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_wb_gather(const WbLaunch& a, hipStream_t st) {
  if (a.b1 <= a.b0) return hipSuccess;
  hipLaunchKernelGGL(k_wb_gather, dim3((unsigned)(a.b1 - a.b0)), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

}  // namespace emb
