// Host runtime of the embedding library: table build from a prebuilt key set, the host image that
// is flashed to HBM in one copy per PASS, validation, write-back/export, and the C ABI.
//
// The table is prepared off-GPU and copied in bulk, with no insert on the device (Tencent PCG GPU
// training talk, flash paragraph of "optimisations of each stage"); keys carry the field id in
// their high 16 bits so all fields share one table (same talk, unified hash table paragraph).
#include "emb.h"

#include <hip/hip_runtime_api.h>
#include <sys/mman.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <new>
#include <numeric>
#include <string>
#include <thread>
#include <vector>

#include "emb_internal.h"

using namespace emb;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

// A failed HIP call also leaves its code as the thread's "last error", which the next caller to
// ask (torch, after its own successful calls) would take as its own failure; clear it here, since
// the code travels back through the return value and emb_last_error().
int hip_fail(hipError_t e, const char* what) {
  (void)hipGetLastError();
  return fail(EMB_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Host worker threads: the hardware's count, capped at 32 and at OMP_NUM_THREADS when it is set
// (the usual way a job states its CPU share).
int n_threads() {
  static const int n = [] {
    unsigned h = std::thread::hardware_concurrency();
    if (h == 0) h = 4;
    h = std::min(h, 32u);
    if (const char* e = std::getenv("OMP_NUM_THREADS")) {
      const long v = std::strtol(e, nullptr, 10);
      if (v > 0) h = std::min(h, (unsigned)v);
    }
    return (int)h;
  }();
  return n;
}

// Run fn(begin, end) over [0, n) split across threads.
template <typename Fn>
void parallel_for(size_t n, Fn fn) {
  const int T = n < 65536 ? 1 : n_threads();
  if (T == 1) {
    fn((size_t)0, n);
    return;
  }
  std::vector<std::thread> th;
  const size_t chunk = (n + T - 1) / T;
  for (int t = 0; t < T; ++t) {
    const size_t b = (size_t)t * chunk, e = std::min(n, b + chunk);
    if (b >= e) break;
    th.emplace_back([=] { fn(b, e); });
  }
  for (auto& x : th) x.join();
}

// fp32 -> fp16 bits, round to nearest even, subnormals kept (from the IEEE-754 binary16 format).
uint16_t f32_to_f16(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u) return (uint16_t)(sign | 0x7C00u | (ax > 0x7F800000u ? 0x200u : 0u));
  const uint32_t e = ax >> 23;
  if (e >= 113) {  // normal half range or overflow
    uint32_t r = ((e - 112) << 10) | ((ax >> 13) & 0x3FFu);
    const uint32_t rb = (ax >> 12) & 1u, sticky = ax & 0xFFFu;
    if (rb && (sticky || (r & 1u))) ++r;
    if (r >= 0x7C00u) r = 0x7C00u;
    return (uint16_t)(sign | r);
  }
  if (e < 102) return (uint16_t)sign;  // below half the smallest subnormal
  const uint32_t m = (ax & 0x7FFFFFu) | 0x800000u;
  const int s = 126 - (int)e;  // 14..24
  uint32_t r = m >> s;
  const uint32_t rb = (m >> (s - 1)) & 1u, sticky = m & ((1u << (s - 1)) - 1u);
  if (rb && (sticky || (r & 1u))) ++r;
  return (uint16_t)(sign | r);
}

float f16_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu, x;
  if (e == 0) {
    if (m == 0) {
      x = sign;
    } else {
      int sh = 0;
      while (!(m & 0x400u)) { m <<= 1; ++sh; }
      m &= 0x3FFu;
      x = sign | ((uint32_t)(113 - sh) << 23) | (m << 13);
    }
  } else if (e == 31) {
    x = sign | 0x7F800000u | (m << 13);
  } else {
    x = sign | ((e + 112) << 23) | (m << 13);
  }
  float f;
  std::memcpy(&f, &x, 4);
  return f;
}

struct Entry {
  uint64_t key;
  uint32_t home;
  uint32_t idx;  // position in the caller's key list
};

bool entry_less(const Entry& a, const Entry& b) {
  return a.home != b.home ? a.home < b.home : a.key < b.key;
}

// Sort by (home, key): partition by home range, then sort the parts in parallel.
void sort_entries(std::vector<Entry>& v, uint32_t n_home) {
  const size_t n = v.size();
  const int T = n < 200000 ? 1 : n_threads();
  if (T == 1) {
    std::sort(v.begin(), v.end(), entry_less);
    return;
  }
  const int P = T * 8;
  auto part_of = [&](uint32_t h) { return (int)(((uint64_t)h * (uint64_t)P) / (uint64_t)n_home); };
  std::vector<std::vector<size_t>> cnt(T, std::vector<size_t>(P + 1, 0));
  const size_t chunk = (n + T - 1) / T;
  {
    std::vector<std::thread> th;
    for (int t = 0; t < T; ++t)
      th.emplace_back([&, t] {
        const size_t b = (size_t)t * chunk, e = std::min(n, b + chunk);
        for (size_t i = b; i < e; ++i) ++cnt[t][part_of(v[i].home)];
      });
    for (auto& x : th) x.join();
  }
  std::vector<size_t> pstart(P + 1, 0);
  std::vector<std::vector<size_t>> pos(T, std::vector<size_t>(P, 0));
  size_t run = 0;
  for (int p = 0; p < P; ++p) {
    pstart[p] = run;
    for (int t = 0; t < T; ++t) {
      pos[t][p] = run;
      run += cnt[t][p];
    }
  }
  pstart[P] = run;
  std::vector<Entry> out(n);
  {
    std::vector<std::thread> th;
    for (int t = 0; t < T; ++t)
      th.emplace_back([&, t] {
        const size_t b = (size_t)t * chunk, e = std::min(n, b + chunk);
        for (size_t i = b; i < e; ++i) out[pos[t][part_of(v[i].home)]++] = v[i];
      });
    for (auto& x : th) x.join();
  }
  std::atomic<int> next{0};
  {
    std::vector<std::thread> th;
    for (int t = 0; t < T; ++t)
      th.emplace_back([&] {
        for (int p; (p = next.fetch_add(1)) < P;)
          std::sort(out.begin() + pstart[p], out.begin() + pstart[p + 1], entry_less);
      });
    for (auto& x : th) x.join();
  }
  v.swap(out);
}

}  // namespace

struct EmbTable {
  // descriptor
  int32_t F = 0;
  std::vector<int32_t> dim, col, gran;
  int32_t row_dtype = EMB_F32, has_master = 0, n_tables = 1, flags = 0;
  double lf = 0.5;
  float acc_init = 0.f;
  int32_t granule = 1, var_dim = 0, max_dim = 0, out_width = 0;
  std::vector<int32_t> gsl;          // per field: log2 of the lanes (16-byte slices) of its rows
  int32_t classed = 0, cls_shift = 0;
  size_t elem_bytes = 4;
  // layout
  struct Sub {
    uint64_t n_keys = 0, n_home = 1, n_buckets = 0, bucket_base = 0;
    uint32_t rowref_base = 0;
  } sub[2];
  uint64_t n_keys = 0, total_buckets = 0, total_elems = 0;
  uint32_t rowref_space = 0;
  size_t off_keys = 0, off_rows = 0, off_acc = 0, off_master = 0, off_linear = 0, off_meta = 0;
  size_t arena_bytes = 0;
  int32_t ftrl = 0;  // the table keeps the FTRL linear state z
  size_t off_touched = 0, touched_words = 0;  // bitmap of rowref units updated since the flash
  size_t off_pstat = 0;  // partial probe statistics (kStatSlots x 4 words, zero in the image)
  std::vector<uint64_t> dirty;  // host: units written back by pass_writeback_touched since cleared
  uint8_t* image = nullptr;
  bool pinned = false;
  // pageable images move through two pinned bounce buffers (host copy of one chunk overlaps the
  // DMA of the other); allocated at the first such copy, null when pinning failed
  static constexpr size_t kBounce = 256u << 20;
  uint8_t* bounce[2] = {nullptr, nullptr};
  hipEvent_t bounce_ev[2] = {nullptr, nullptr};
  bool bounce_tried = false;
  // probe statistics the forward adds to (device, caller-owned), null when off
  unsigned long long* probe_stats = nullptr;
  // EMB_VALIDATE=1: one device word the validation kernel reports into (allocated at first use)
  uint32_t* d_vflag = nullptr;
  std::vector<uint64_t> row_keys;  // keys in rowref order
  std::vector<uint32_t> row_ref;   // their rowrefs (ascending)
  std::vector<uint32_t> row_of_key;  // position in row_keys of the i-th key given at create
  double mean_disp = 0;
  uint64_t max_disp = 0;
  // device
  uint8_t* d_arena = nullptr;
  bool flashed = false;
  // the workspace the last sparse_bwd_dedup sorted, for the one apply call it enables
  struct Dedup {
    const void* ws = nullptr;
    int64_t n_bags = -1, nnz = -1;
  } dedup;
  Timing timing;

  uint64_t* keys_img() { return reinterpret_cast<uint64_t*>(image + off_keys); }
  const uint64_t* keys_img() const { return reinterpret_cast<const uint64_t*>(image + off_keys); }

  DevDesc dev() const {
    DevDesc d{};
    for (int t = 0; t < 2; ++t) {
      const int s = t < n_tables ? t : 0;
      d.tab[t].buckets = reinterpret_cast<const uint64_t*>(d_arena + off_keys) +
                         sub[s].bucket_base * kWordsPerBucket;
      d.tab[t].n_home = (uint32_t)sub[s].n_home;
      d.tab[t].n_buckets = (uint32_t)sub[s].n_buckets;
    }
    d.n_tables = n_tables;
    d.n_fields = F;
    d.granule = granule;
    d.var_dim = var_dim;
    d.fixed_dim = dim[0];
    d.max_dim = max_dim;
    d.out_width = out_width;
    d.row_f16 = row_dtype == EMB_F16;
    d.has_master = has_master;
    d.rows = d_arena + off_rows;
    d.acc = reinterpret_cast<float*>(d_arena + off_acc);
    d.master = has_master ? reinterpret_cast<float*>(d_arena + off_master) : nullptr;
    d.linear = ftrl ? reinterpret_cast<float*>(d_arena + off_linear) : nullptr;
    const int32_t* meta = reinterpret_cast<const int32_t*>(d_arena + off_meta);
    d.fdim = meta;
    d.fcol = meta + F;
    d.fgran = meta + 2 * F;
    d.fgsl = meta + 3 * F;
    d.classed = classed;
    d.cls_shift = cls_shift;
    d.touched = (flags & EMB_FLAG_TRACK_TOUCHED)
                    ? reinterpret_cast<uint32_t*>(d_arena + off_touched) : nullptr;
    d.pstat = reinterpret_cast<unsigned long long*>(d_arena + off_pstat);
    d.rowref_space = rowref_space;
    // division by the field count as a multiply and shift (exact for dividends below 2^31)
    int l = 0;
    while ((1u << l) < (uint32_t)F) ++l;
    d.fdiv_s = 31 + l;
    d.fdiv_m = (uint32_t)(((1ull << d.fdiv_s) + (uint64_t)F - 1) / (uint64_t)F);
    return d;
  }

  // Host probe over the image: the same scan the device runs.
  bool probe(uint64_t key, uint32_t* rr, int64_t* slot) const {
    if (key == kEmpty || (int64_t)(key >> 48) >= F) return false;
    const int t = (n_tables == 2) ? (int)(key & 1) : 0;
    const Sub& s = sub[t];
    const uint32_t home = home_slot(mix64(key), (uint32_t)s.n_home);
    uint64_t b = home / kKeysPerBucket;
    uint32_t l0 = home - (uint32_t)b * kKeysPerBucket;
    const uint64_t* kb = keys_img() + s.bucket_base * kWordsPerBucket;
    for (; b < s.n_buckets; ++b, l0 = 0) {
      const uint64_t* w = kb + b * kWordsPerBucket;
      for (uint32_t l = l0; l < (uint32_t)kKeysPerBucket; ++l) {
        if (w[l] == key) {
          uint32_t r = (uint32_t)w[15];
          for (uint32_t q = 0; q < l; ++q)
            if (w[q] != kEmpty) r += (uint32_t)gran[(int)(w[q] >> 48)];
          *rr = r;
          *slot = (int64_t)(b * kKeysPerBucket + l);
          return true;
        }
        if (w[l] == kEmpty) return false;
      }
    }
    return false;
  }

  bool ensure_bounce() {
    if (bounce_tried) return bounce[1] != nullptr;
    bounce_tried = true;
    for (int i = 0; i < 2; ++i) {
      if (hipHostMalloc(reinterpret_cast<void**>(&bounce[i]), kBounce, 0) != hipSuccess ||
          hipEventCreateWithFlags(&bounce_ev[i], hipEventDisableTiming) != hipSuccess) {
        (void)hipGetLastError();
        release_bounce();
        return false;
      }
    }
    return true;
  }
  void release_bounce() {
    for (int i = 0; i < 2; ++i) {
      if (bounce_ev[i]) {
        (void)hipEventSynchronize(bounce_ev[i]);
        (void)hipEventDestroy(bounce_ev[i]);
        bounce_ev[i] = nullptr;
      }
      if (bounce[i]) (void)hipHostFree(bounce[i]);
      bounce[i] = nullptr;
    }
  }

  ~EmbTable() {
    release_bounce();
    if (d_vflag) (void)hipFree(d_vflag);
    for (auto& r : timing.pool) {
      (void)hipEventDestroy(r.a);
      (void)hipEventDestroy(r.b);
    }
    if (image) {
      if (pinned) (void)hipHostFree(image);
      else std::free(image);
    }
  }
};

// Host copy spread over threads (a pageable image chunk into or out of a bounce buffer).
void par_copy(uint8_t* dst, const uint8_t* src, size_t n) {
  const int T = std::max(1, std::min(n_threads(), (int)(n >> 22)));  // at least 4 MiB a thread
  const size_t part = ((n + T - 1) / T + 4095) & ~(size_t)4095;
  std::vector<std::thread> th;
  for (int i = 0; i < T; ++i) {
    const size_t o = (size_t)i * part;
    if (o >= n) break;
    th.emplace_back([=] { std::memcpy(dst + o, src + o, std::min(part, n - o)); });
  }
  for (auto& x : th) x.join();
}

// Host image -> device through the bounce buffers: chunk k is copied into buffer k % 2 once the
// DMA that last read that buffer has finished, then its DMA is enqueued on the stream.
hipError_t flash_bounced(EmbTable* t, uint8_t* d, const uint8_t* h, size_t n, hipStream_t st) {
  const size_t C = EmbTable::kBounce;
  for (size_t o = 0, k = 0; o < n; o += C, ++k) {
    const int b = (int)(k & 1);
    const size_t len = std::min(C, n - o);
    hipError_t e = hipEventSynchronize(t->bounce_ev[b]);
    if (e != hipSuccess) return e;
    par_copy(t->bounce[b], h + o, len);
    e = hipMemcpyAsync(d + o, t->bounce[b], len, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return e;
    e = hipEventRecord(t->bounce_ev[b], st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Device -> host image through the bounce buffers: the DMA of chunk k + 1 runs while chunk k is
// copied out of its buffer.
hipError_t writeback_bounced(EmbTable* t, uint8_t* h, const uint8_t* d, size_t n, hipStream_t st) {
  const size_t C = EmbTable::kBounce;
  const size_t chunks = (n + C - 1) / C;
  hipError_t e = hipSuccess;
  auto issue = [&](size_t k) {
    const int b = (int)(k & 1);
    const size_t o = k * C, len = std::min(C, n - o);
    hipError_t r = hipMemcpyAsync(t->bounce[b], d + o, len, hipMemcpyDeviceToHost, st);
    if (r == hipSuccess) r = hipEventRecord(t->bounce_ev[b], st);
    return r;
  };
  if (chunks) e = issue(0);
  for (size_t k = 0; k < chunks && e == hipSuccess; ++k) {
    if (k + 1 < chunks) e = issue(k + 1);
    if (e != hipSuccess) break;
    const int b = (int)(k & 1);
    e = hipEventSynchronize(t->bounce_ev[b]);
    if (e != hipSuccess) break;
    const size_t o = k * C;
    par_copy(h + o, t->bounce[b], std::min(C, n - o));
  }
  return e;
}

extern "C" {

const char* emb_last_error(void) { return g_err.c_str(); }

namespace {
// Device resources for building the layout on the GPU (table_create_on_device).
struct DevBuild {
  uint8_t* ws;
  size_t ws_bytes;
  hipStream_t st;
};

// Workspace carve-up of the device build for n keys.  The sort region holds the radix sort's
// buffers for any sort-key space: the widest plan plus room for 9-bit digits on every tile.
struct BuildPlan {
  size_t off_keys, off_sort, sort_bytes, off_gran, off_bmax, off_bsum, off_misc, off_buckets, bytes;
  int64_t max_blocks;
  uint64_t max_buckets;
};
BuildPlan plan_build(int64_t n, uint64_t bucket_bound, int F) {
  BuildPlan b{};
  const BwdPlan wide = plan_bwd(n, 0xFFFFFFFFu, 8, 0, 0);
  b.sort_bytes = wide.bytes + 4 * 513 * ((size_t)wide.tiles + (size_t)wide.groups + 2) + 4096;
  size_t o = 0;
  b.off_keys = o; o = align256(o + 8 * (size_t)n);
  b.off_sort = o; o = align256(o + b.sort_bytes);
  b.off_gran = o; o = align256(o + 4 * (size_t)F);
  b.max_blocks = (n + (int64_t)kBuildTile - 1) / ((int64_t)kBuildTile) + 1;
  b.off_bmax = o; o = align256(o + 8 * (size_t)(b.max_blocks + 1));
  b.off_bsum = o; o = align256(o + 4 * (size_t)(b.max_blocks + 1));
  b.off_misc = o; o = align256(o + 64);
  b.max_buckets = bucket_bound;
  b.off_buckets = o; o = align256(o + 128 * (size_t)bucket_bound);
  b.bytes = o;
  return b;
}
// Buckets a table of n keys can need at most: its home slots plus one slot per key of overflow,
// plus the terminator; for two tables, both.
uint64_t bucket_bound(int64_t n, double lf, int n_tables) {
  const uint64_t nh = (uint64_t)std::ceil((double)n / lf) + 2 * (uint64_t)n_tables;
  return (nh + (uint64_t)n + (uint64_t)kKeysPerBucket * n_tables) / kKeysPerBucket + 2 * (uint64_t)n_tables;
}

// The ordered linear-probing layout computed on the GPU: same slots, rowrefs and buckets as the
// host builder.  On return `order` holds the caller index of each key in rowref order and the
// bucket words sit in the workspace at d_buckets.
int device_layout(EmbTable* T, const uint64_t* K, size_t N, const DevBuild& db,
                  std::vector<uint32_t>& order, uint64_t*& d_buckets, double& disp_sum) {
  const uint64_t nh0 = T->sub[0].n_home, nh1 = T->n_tables == 2 ? T->sub[1].n_home : 0;
  if (nh0 + nh1 >= 0xFFFFFFF0ull) return fail(EMB_ERANGE, "too many home slots for the device build");
  const BuildPlan bp = plan_build((int64_t)N, bucket_bound((int64_t)N, T->lf, T->n_tables), T->F);
  if (db.ws_bytes < bp.bytes) return fail(EMB_ENOSPACE, "workspace smaller than table_build_workspace_bytes()");
  uint8_t* ws = db.ws;
  hipStream_t st = db.st;
  BuildArgs a{};
  a.keys = reinterpret_cast<const uint64_t*>(ws + bp.off_keys);
  a.n = (int64_t)N;
  a.n_tables = T->n_tables;
  a.n_home0 = (uint32_t)nh0;
  a.n_home1 = (uint32_t)nh1;
  a.gran = reinterpret_cast<const int32_t*>(ws + bp.off_gran);
  uint8_t* sws = ws + bp.off_sort;
  const BwdPlan sp = plan_bwd((int64_t)N, (uint32_t)(nh0 + nh1), 8, 0, 0);
  if (sp.bytes > bp.sort_bytes) return fail(EMB_ENOSPACE, "device build: sort plan exceeds its region");
  a.skey = reinterpret_cast<uint32_t*>(sws + sp.off_ka);
  a.sval = reinterpret_cast<uint32_t*>(sws + sp.off_va);
  uint32_t* misc = reinterpret_cast<uint32_t*>(ws + bp.off_misc);
  a.dup = misc;
  a.disp = reinterpret_cast<unsigned long long*>(misc + 2);
  a.bmax = reinterpret_cast<int64_t*>(ws + bp.off_bmax);
  a.bsum = reinterpret_cast<uint32_t*>(ws + bp.off_bsum);
  a.buckets = reinterpret_cast<uint64_t*>(ws + bp.off_buckets);
  hipError_t e = hipMemsetAsync(misc, 0, 64, st);
  if (e == hipSuccess && N) e = hipMemcpyAsync(ws + bp.off_keys, K, 8 * N, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipMemcpyAsync(ws + bp.off_gran, T->gran.data(), 4 * (size_t)T->F, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = launch_build_homes(a, st);
  uint32_t *ks = a.skey, *vs = a.sval;
  if (e == hipSuccess) e = launch_build_sort(a, sp, sws, &ks, &vs, st);
  a.sk = ks;
  a.sv = vs;
  if (e == hipSuccess) e = launch_build_ties(a, st);
  uint32_t dup = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&dup, a.dup, 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "device layout build (sort)");
  if (dup) return fail(EMB_EDUPKEY, "duplicate key in the prebuilt key set");

  // per table: slot and unit scans, then the table's bucket count and bases
  const size_t n0 = T->sub[0].n_keys;
  int64_t seg[2][2] = {{0, (int64_t)n0}, {(int64_t)n0, (int64_t)N}};
  uint64_t rr = 0, bb = 0;
  int64_t lastm[2] = {0, 0};
  for (int t = 0; t < T->n_tables; ++t) {
    EmbTable::Sub& s = T->sub[t];
    BuildArgs g = a;
    g.s0 = seg[t][0];
    g.s1 = seg[t][1];
    g.home_base = t ? (uint32_t)nh0 : 0u;
    g.blocks = (g.s1 - g.s0 + (int64_t)kBuildTile - 1) / ((int64_t)kBuildTile);
    int64_t tot_m = 0;
    uint32_t tot_u = 0;
    if (g.blocks > 0) {
      e = launch_build_scan(g, st);
      if (e == hipSuccess) e = hipMemcpyAsync(&tot_m, g.bmax + g.blocks, 8, hipMemcpyDeviceToHost, st);
      if (e == hipSuccess) e = hipMemcpyAsync(&tot_u, g.bsum + g.blocks, 4, hipMemcpyDeviceToHost, st);
      if (e == hipSuccess) e = hipStreamSynchronize(st);
      if (e != hipSuccess) return hip_fail(e, "device layout build (scan)");
    }
    lastm[t] = tot_m;
    const uint64_t nt = (uint64_t)(g.s1 - g.s0);
    const uint64_t last = nt ? (nt - 1) + (uint64_t)tot_m : 0;
    const uint64_t span = std::max<uint64_t>(s.n_home, nt ? last + 1 : 0);
    s.n_buckets = (span + kKeysPerBucket - 1) / kKeysPerBucket + 1;
    if (s.n_buckets > 0xFFFFFFF0ull) return fail(EMB_ERANGE, "table too large");
    s.bucket_base = bb;
    bb += s.n_buckets;
    if (bb > 0xFFFFFFFFull) return fail(EMB_ERANGE, "bucket arrays exceed 2^32 buckets");
    s.rowref_base = (uint32_t)rr;
    rr += tot_u;
    if (rr >= 0xFFFFFFFFull) return fail(EMB_ERANGE, "rowref space exceeds 32 bits");
  }
  if (bb > bp.max_buckets) return fail(EMB_ERANGE, "device build: bucket bound exceeded");
  T->total_buckets = bb;
  T->rowref_space = (uint32_t)rr;
  // every key word starts EMPTY; then keys, prefix words and the tail of each table
  e = hipMemsetAsync(a.buckets, 0xFF, 128 * (size_t)bb, st);
  for (int t = 0; t < T->n_tables && e == hipSuccess; ++t) {
    EmbTable::Sub& s = T->sub[t];
    BuildArgs g = a;
    g.s0 = seg[t][0];
    g.s1 = seg[t][1];
    g.home_base = t ? (uint32_t)nh0 : 0u;
    g.blocks = (g.s1 - g.s0 + (int64_t)kBuildTile - 1) / ((int64_t)kBuildTile);
    if (g.blocks > 0) e = launch_build_scan(g, st);  // the block prefixes again (same values)
    const uint64_t nt = (uint64_t)(g.s1 - g.s0);
    g.bucket_base = s.bucket_base;
    g.n_buckets = s.n_buckets;
    g.rowref_base = s.rowref_base;
    g.tail_from = nt ? ((nt - 1) + (uint64_t)lastm[t]) / kKeysPerBucket + 1 : 0;
    g.tail_value = (uint32_t)(t + 1 < T->n_tables ? T->sub[t + 1].rowref_base : rr);
    if (e == hipSuccess) e = launch_build_place(g, st);
  }
  order.resize(N);
  unsigned long long disp[2] = {0, 0};
  if (e == hipSuccess && N) e = hipMemcpyAsync(order.data(), a.sv, 4 * N, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipMemcpyAsync(disp, a.disp, 16, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "device layout build (place)");
  disp_sum = (double)disp[0];
  T->max_disp = disp[1];
  d_buckets = a.buckets;
  return EMB_OK;
}

int create_impl(const EmbTableDesc* desc, const int64_t* keys, int64_t n_keys, const void* rows,
                const float* acc, const float* master, const DevBuild* db, EmbTable** out);
}  // namespace

int table_create_from_prebuilt(const EmbTableDesc* desc, const int64_t* keys, int64_t n_keys,
                               const void* rows, const float* acc, const float* master,
                               EmbTable** out) {
  return create_impl(desc, keys, n_keys, rows, acc, master, nullptr, out);
}

int table_build_workspace_bytes(const EmbTableDesc* desc, int64_t n_keys, size_t* bytes) {
  if (!desc || !bytes) return fail(EMB_EINVAL, "null argument");
  if (n_keys < 0 || n_keys >= (1ll << 31)) return fail(EMB_ERANGE, "the device build takes fewer than 2^31 keys");
  if (!(desc->load_factor > 0.0 && desc->load_factor <= 1.0))
    return fail(EMB_EINVAL, "load_factor must be in (0, 1]");
  if (desc->n_fields < 1 || desc->n_fields > kMaxFields) return fail(EMB_EINVAL, "n_fields must be in [1, 65535]");
  const int nt = desc->n_tables == 2 ? 2 : 1;
  *bytes = plan_build(n_keys, bucket_bound(n_keys, desc->load_factor, nt), desc->n_fields).bytes;
  return EMB_OK;
}

int table_create_on_device(const EmbTableDesc* desc, const int64_t* keys, int64_t n_keys,
                           void* d_ws, size_t ws_bytes, emb_stream_t stream, EmbTable** out) {
  if (!d_ws || reinterpret_cast<uintptr_t>(d_ws) % 256)
    return fail(EMB_EINVAL, "workspace must be non-null and 256-byte aligned");
  if (n_keys >= (1ll << 31)) return fail(EMB_ERANGE, "the device build takes fewer than 2^31 keys");
  DevBuild db{static_cast<uint8_t*>(d_ws), ws_bytes, static_cast<hipStream_t>(stream)};
  return create_impl(desc, keys, n_keys, nullptr, nullptr, nullptr, &db, out);
}

namespace {
int create_impl(const EmbTableDesc* desc, const int64_t* keys, int64_t n_keys, const void* rows,
                const float* acc, const float* master, const DevBuild* db, EmbTable** out) {
  if (!desc || !out) return fail(EMB_EINVAL, "null descriptor or output pointer");
  *out = nullptr;
  if (desc->n_fields < 1 || desc->n_fields > kMaxFields)
    return fail(EMB_EINVAL, "n_fields must be in [1, 65535]");
  if (!desc->field_dim) return fail(EMB_EINVAL, "null field_dim");
  if (desc->row_dtype != EMB_F32 && desc->row_dtype != EMB_F16)
    return fail(EMB_EINVAL, "row_dtype must be EMB_F32 or EMB_F16");
  if (desc->has_master && desc->row_dtype != EMB_F16)
    return fail(EMB_EINVAL, "a master copy needs fp16 rows");
  if (desc->n_tables != 1 && desc->n_tables != 2) return fail(EMB_EINVAL, "n_tables must be 1 or 2");
  if (!(desc->load_factor > 0.0 && desc->load_factor <= 1.0))
    return fail(EMB_EINVAL, "load_factor must be in (0, 1]");
  if (n_keys < 0 || n_keys > 0xFFFFFFF0ll) return fail(EMB_ERANGE, "n_keys out of range");
  if (n_keys > 0 && !keys) return fail(EMB_EINVAL, "null keys");

  EmbTable* T = new (std::nothrow) EmbTable();
  if (!T) return fail(EMB_ENOMEM, "out of host memory");
  std::unique_ptr<EmbTable> guard(T);
  T->F = desc->n_fields;
  T->row_dtype = desc->row_dtype;
  T->has_master = desc->has_master ? 1 : 0;
  T->ftrl = (desc->flags & EMB_FLAG_FTRL) ? 1 : 0;
  T->n_tables = desc->n_tables;
  T->lf = desc->load_factor;
  T->acc_init = desc->acc_init;
  T->flags = desc->flags;
  T->elem_bytes = desc->row_dtype == EMB_F16 ? 2 : 4;
  T->dim.assign(desc->field_dim, desc->field_dim + desc->n_fields);
  int g = 0;
  int64_t width = 0;
  for (int f = 0; f < T->F; ++f) {
    const int d = T->dim[f];
    if (d < 8 || d > kMaxDim || d % 8) return fail(EMB_EINVAL, "field dims must be multiples of 8 in [8, 256]");
    g = std::gcd(g, d);
    T->max_dim = std::max(T->max_dim, d);
    T->col.push_back((int32_t)width);
    width += d;
    if (d != T->dim[0]) T->var_dim = 1;
  }
  if (width > (1 << 30)) return fail(EMB_ERANGE, "sum of field dims too large");
  T->granule = g;
  T->out_width = (int32_t)width;
  for (int f = 0; f < T->F; ++f) T->gran.push_back(T->dim[f] / g);

  // validate keys and route them to tables
  const uint64_t* K = reinterpret_cast<const uint64_t*>(keys);
  const size_t N = (size_t)n_keys;
  T->n_keys = N;
  std::atomic<int> bad{0};
  std::vector<uint64_t> tcount(2, 0);
  {
    std::vector<std::vector<uint64_t>> part(64, std::vector<uint64_t>(2, 0));
    std::atomic<int> slot{0};
    parallel_for(N, [&](size_t b, size_t e) {
      const int my = slot.fetch_add(1);
      uint64_t c0 = 0, c1 = 0;
      for (size_t i = b; i < e; ++i) {
        const uint64_t k = K[i];
        if (k == kEmpty) bad.store(1);
        else if ((int64_t)(k >> 48) >= T->F) { int z = 0; bad.compare_exchange_strong(z, 2); }
        if (T->n_tables == 2 && (k & 1)) ++c1; else ++c0;
      }
      part[my % 64][0] += c0;
      part[my % 64][1] += c1;
    });
    for (auto& p : part) { tcount[0] += p[0]; tcount[1] += p[1]; }
  }
  if (bad.load() == 1) return fail(EMB_ESENTINEL, "a key equals the EMPTY marker (all bits set)");
  if (bad.load() == 2) return fail(EMB_ERANGE, "a key's field id is >= n_fields");

  // input row offsets (elements) in key order; implicit (i * D) when every field has width D
  std::vector<uint64_t> in_off;
  if (T->var_dim) {
    in_off.assign(N + 1, 0);
    for (size_t i = 0; i < N; ++i) in_off[i + 1] = in_off[i] + (uint64_t)T->dim[(int)(K[i] >> 48)];
    T->total_elems = in_off[N];
  } else {
    T->total_elems = (uint64_t)N * (uint64_t)T->dim[0];
  }
  const uint64_t fixed_d = (uint64_t)T->dim[0];
  auto src_off = [&](size_t i) { return T->var_dim ? in_off[i] : (uint64_t)i * fixed_d; };

  // per table: homes, sort by (home, key), place, count buckets
  std::vector<Entry> ent[2];
  uint64_t rr_total = 0;
  double disp_sum = 0;
  std::vector<uint64_t> slot_of[2];
  for (int t = 0; t < T->n_tables; ++t) {
    EmbTable::Sub& s = T->sub[t];
    s.n_keys = tcount[t];
    const double nh = std::ceil((double)s.n_keys / T->lf);
    if (nh > 4294967295.0 - 64) return fail(EMB_ERANGE, "too many home slots for one table");
    s.n_home = std::max<uint64_t>(1, (uint64_t)nh);
    if (!db) ent[t].resize(s.n_keys);
  }
  std::vector<uint32_t> dev_order;   // device build: caller index of each key in rowref order
  uint64_t* d_buckets = nullptr;
  if (db) {
    const int rc = device_layout(T, K, N, *db, dev_order, d_buckets, disp_sum);
    if (rc) return rc;
    rr_total = T->rowref_space;
  } else {
    size_t p0 = 0, p1 = 0;
    for (size_t i = 0; i < N; ++i) {
      const int t = (T->n_tables == 2 && (K[i] & 1)) ? 1 : 0;
      Entry& en = ent[t][t ? p1++ : p0++];
      en.key = K[i];
      en.idx = (uint32_t)i;
    }
  for (int t = 0; t < T->n_tables; ++t) {
    EmbTable::Sub& s = T->sub[t];
    std::vector<Entry>& E = ent[t];
    const uint32_t nh = (uint32_t)s.n_home;
    parallel_for(E.size(), [&](size_t b, size_t e) {
      for (size_t i = b; i < e; ++i) E[i].home = home_slot(mix64(E[i].key), nh);
    });
    sort_entries(E, nh);
    for (size_t i = 1; i < E.size(); ++i)
      if (E[i].key == E[i - 1].key) return fail(EMB_EDUPKEY, "duplicate key in the prebuilt key set");
    slot_of[t].resize(E.size());
    uint64_t last = 0;
    for (size_t i = 0; i < E.size(); ++i) {
      const uint64_t sl = i == 0 ? E[i].home : std::max<uint64_t>(E[i].home, last + 1);
      slot_of[t][i] = sl;
      last = sl;
      disp_sum += (double)(sl - E[i].home);
      T->max_disp = std::max<uint64_t>(T->max_disp, sl - E[i].home);
    }
    const uint64_t span = std::max<uint64_t>(s.n_home, E.empty() ? 0 : last + 1);
    s.n_buckets = (span + kKeysPerBucket - 1) / kKeysPerBucket + 1;  // + an all-empty terminator
    if (s.n_buckets > 0xFFFFFFF0ull) return fail(EMB_ERANGE, "table too large");
    s.bucket_base = T->total_buckets;
    T->total_buckets += s.n_buckets;
    if (T->total_buckets > 0xFFFFFFFFull) return fail(EMB_ERANGE, "bucket arrays exceed 2^32 buckets");
    s.rowref_base = (uint32_t)rr_total;
    for (const Entry& en : E) rr_total += (uint64_t)T->gran[(int)(en.key >> 48)];
    if (rr_total >= 0xFFFFFFFFull) return fail(EMB_ERANGE, "rowref space exceeds 32 bits");
  }
  }  // host layout
  T->rowref_space = (uint32_t)rr_total;
  // width classes: log2 of the 16-byte lanes a row takes; the backward sorts mixed-width tables
  // by (class, rowref) when the classes fit above the rowref bits and the first radix digit
  // (at most 9 bits) stays below them
  {
    const int epl = T->row_dtype == EMB_F16 ? 8 : 4;
    int cmin = 99, cmax = -1;
    for (int f = 0; f < T->F; ++f) {
      const int lanes = (T->dim[f] + epl - 1) / epl;
      int g = 0;
      while ((1 << g) < lanes) ++g;
      T->gsl.push_back(g);
      cmin = std::min(cmin, g);
      cmax = std::max(cmax, g);
    }
    int rbits = 0;
    while (rbits < 32 && T->rowref_space > 1 && ((uint64_t)(T->rowref_space - 1) >> rbits) != 0) ++rbits;
    if (cmax > cmin && rbits >= 9 && rbits + 3 <= 31) {
      T->classed = 1;
      T->cls_shift = rbits;
    }
  }
  T->mean_disp = N ? disp_sum / (double)N : 0.0;

  // image layout = arena layout.  On mixed-width tables each state array is followed by one
  // widest row of zeros: a rowref that names a row narrower than its bag's field (caller-supplied
  // rowrefs from another batch) then updates elements of the wrong rows, or the pad, but never
  // the next array or the field metadata the kernels index with.
  const size_t eb = T->elem_bytes;
  const size_t pad = T->var_dim ? (size_t)T->max_dim : 0;
  const size_t EP = T->total_elems + pad;
  T->off_keys = 0;
  T->off_rows = align256(T->total_buckets * 128);
  T->off_acc = align256(T->off_rows + EP * eb);
  T->off_master = align256(T->off_acc + EP * 4);
  T->off_linear = align256(T->off_master + (T->has_master ? EP * 4 : 0));
  T->off_meta = align256(T->off_linear + (T->ftrl ? EP * 4 : 0));
  // 4 KiB of tail padding: kernels read row 0 (+ lane offset) in place of a masked-off row, which
  // must stay inside the arena even for an empty table
  T->off_touched = align256(T->off_meta + 4 * 4 * (size_t)T->F);
  T->touched_words = (T->flags & EMB_FLAG_TRACK_TOUCHED) ? ((size_t)T->rowref_space + 31) / 32 : 0;
  T->off_pstat = align256(T->off_touched + 4 * T->touched_words);
  T->arena_bytes = align256(T->off_pstat + 32 * (size_t)kStatSlots) + 4096;
  if (T->flags & EMB_FLAG_PINNED_STAGING) {
    hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&T->image), T->arena_bytes, 0);
    if (e != hipSuccess) return hip_fail(e, "hipHostMalloc of the host image");
    T->pinned = true;
  } else {
    // 2 MiB aligned and marked for transparent huge pages: the write-back's scatter and the
    // builder touch the image all over, and 4 KiB pages would make that TLB-bound
    const size_t huge = 2u << 20;
    const size_t bytes = (T->arena_bytes + huge - 1) & ~(huge - 1);
    T->image = static_cast<uint8_t*>(std::aligned_alloc(huge, bytes));
    if (!T->image) return fail(EMB_ENOMEM, "host image allocation failed");
    (void)madvise(T->image, bytes, MADV_HUGEPAGE);  // advice only; ignored where THP is off
  }

  // the alignment gaps between regions and the tail pad hold zeros, so the image (and every
  // arena flashed from it) is a pure function of the table's contents
  {
    const size_t eb0 = T->elem_bytes, E = T->total_elems;
    const size_t ends[7][2] = {
        {T->total_buckets * 128, T->off_rows},
        {T->off_rows + E * eb0, T->off_acc},
        {T->off_acc + E * 4, T->off_master},
        {T->off_master + (T->has_master ? E * 4 : 0), T->off_linear},
        {T->off_linear + (T->ftrl ? E * 4 : 0), T->off_meta},
        {T->off_meta + 16 * (size_t)T->F, T->off_touched},
        {T->off_touched + 4 * T->touched_words, T->arena_bytes}};
    for (const auto& g : ends)
      if (g[1] > g[0]) std::memset(T->image + g[0], 0, g[1] - g[0]);
  }
  // key buckets with per-bucket rowref prefix; per key its rowref
  uint64_t* KB = T->keys_img();
  T->row_keys.resize(N);
  T->row_ref.resize(N);
  std::vector<uint32_t> idx_by_row;
  if (db) {
    // the device built the buckets; rowrefs are the running sum of row units in rowref order
    hipError_t e = hipMemcpyAsync(KB, d_buckets, 128 * (size_t)T->total_buckets,
                                  hipMemcpyDeviceToHost, db->st);
    if (e == hipSuccess) e = hipStreamSynchronize(db->st);
    if (e != hipSuccess) return hip_fail(e, "device layout build (bucket copy)");
    idx_by_row.swap(dev_order);
    const int nt = std::max(1, std::min(n_threads(), (int)(N >> 16)));
    const size_t chunk = (N + nt - 1) / nt;
    std::vector<uint64_t> part((size_t)nt + 1, 0);
    std::vector<std::thread> th;
    for (int c = 0; c < nt; ++c)
      th.emplace_back([&, c] {
        uint64_t u = 0;
        for (size_t r = (size_t)c * chunk; r < std::min(N, (size_t)(c + 1) * chunk); ++r) {
          const uint64_t k = K[idx_by_row[r]];
          T->row_keys[r] = k;
          u += (uint64_t)T->gran[(int)(k >> 48)];
        }
        part[(size_t)c + 1] = u;
      });
    for (auto& x : th) x.join();
    th.clear();
    for (int c = 0; c < nt; ++c) part[(size_t)c + 1] += part[(size_t)c];
    for (int c = 0; c < nt; ++c)
      th.emplace_back([&, c] {
        uint64_t u = part[(size_t)c];
        for (size_t r = (size_t)c * chunk; r < std::min(N, (size_t)(c + 1) * chunk); ++r) {
          T->row_ref[r] = (uint32_t)u;
          u += (uint64_t)T->gran[(int)(T->row_keys[r] >> 48)];
        }
      });
    for (auto& x : th) x.join();
  } else {
  parallel_for(T->total_buckets * kWordsPerBucket, [&](size_t b, size_t e) {
    std::fill(KB + b, KB + e, kEmpty);
  });
  idx_by_row.resize(N);
  size_t rpos = 0;
  for (int t = 0; t < T->n_tables; ++t) {
    EmbTable::Sub& s = T->sub[t];
    uint64_t* kb = KB + s.bucket_base * kWordsPerBucket;
    uint64_t run = s.rowref_base;
    uint64_t next_b = 0;  // next bucket whose prefix is still to be written
    const std::vector<Entry>& E = ent[t];
    for (size_t i = 0; i < E.size(); ++i) {
      const uint64_t sl = slot_of[t][i];
      const uint64_t b = sl / kKeysPerBucket, l = sl % kKeysPerBucket;
      for (; next_b <= b; ++next_b) kb[next_b * kWordsPerBucket + 15] = run;
      kb[b * kWordsPerBucket + l] = E[i].key;
      T->row_keys[rpos] = E[i].key;
      T->row_ref[rpos] = (uint32_t)run;
      idx_by_row[rpos] = E[i].idx;
      ++rpos;
      run += (uint64_t)T->gran[(int)(E[i].key >> 48)];
    }
    for (; next_b < s.n_buckets; ++next_b) kb[next_b * kWordsPerBucket + 15] = run;
    std::vector<Entry>().swap(ent[t]);
    std::vector<uint64_t>().swap(slot_of[t]);
  }
  }  // host layout
  T->row_of_key.resize(N);
  parallel_for(N, [&](size_t b, size_t e) {
    for (size_t r = b; r < e; ++r) T->row_of_key[idx_by_row[r]] = (uint32_t)r;
  });

  // rows, accumulator, master in rowref order
  uint8_t* R = T->image + T->off_rows;
  float* A = reinterpret_cast<float*>(T->image + T->off_acc);
  float* M = T->has_master ? reinterpret_cast<float*>(T->image + T->off_master) : nullptr;
  const uint8_t* rin = static_cast<const uint8_t*>(rows);
  const int f16rows = T->row_dtype == EMB_F16;
  parallel_for(N, [&](size_t b, size_t e) {
    for (size_t r = b; r < e; ++r) {
      const uint32_t i = idx_by_row[r];
      const uint64_t D = (uint64_t)T->dim[(int)(T->row_keys[r] >> 48)];
      const uint64_t dst = (uint64_t)T->row_ref[r] * (uint64_t)T->granule;
      const uint64_t src = src_off(i);
      if (rin) {
        std::memcpy(R + dst * eb, rin + src * eb, D * eb);
      } else if (master && f16rows) {
        uint16_t* h = reinterpret_cast<uint16_t*>(R) + dst;
        for (uint64_t q = 0; q < D; ++q) h[q] = f32_to_f16(master[src + q]);
      } else {
        std::memset(R + dst * eb, 0, D * eb);
      }
      if (acc) std::memcpy(A + dst, acc + src, D * 4);
      else std::fill(A + dst, A + dst + D, T->acc_init);
      if (M) {
        if (master) {
          std::memcpy(M + dst, master + src, D * 4);
        } else {
          const uint16_t* h = reinterpret_cast<const uint16_t*>(R) + dst;
          for (uint64_t q = 0; q < D; ++q) M[dst + q] = f16_to_f32(h[q]);
        }
      }
    }
  });
  // FTRL linear state starts at zero
  if (T->ftrl) {
    uint8_t* L = T->image + T->off_linear;
    parallel_for(T->total_elems, [&](size_t b, size_t e) { std::memset(L + 4 * b, 0, 4 * (e - b)); });
  }
  // the image's bitmap is all clear, so every flash starts with no row marked
  std::memset(T->image + T->off_touched, 0, 4 * T->touched_words);
  int32_t* meta = reinterpret_cast<int32_t*>(T->image + T->off_meta);
  for (int f = 0; f < T->F; ++f) {
    meta[f] = T->dim[f];
    meta[T->F + f] = T->col[f];
    meta[2 * T->F + f] = T->gran[f];
    meta[3 * T->F + f] = T->gsl[f];
  }
  *out = guard.release();
  return EMB_OK;
}
}  // namespace

int table_info(const EmbTable* t, EmbTableInfo* info) {
  if (!t || !info) return fail(EMB_EINVAL, "null argument");
  std::memset(info, 0, sizeof(*info));
  info->arena_bytes = t->arena_bytes;
  info->key_bytes = t->total_buckets * 128;
  info->state_bytes = t->off_meta - t->off_rows;
  info->n_keys = t->n_keys;
  info->total_elems = t->total_elems;
  info->rowref_space = t->rowref_space;
  info->granule = (uint32_t)t->granule;
  for (int s = 0; s < t->n_tables; ++s) {
    info->n_home[s] = t->sub[s].n_home;
    info->n_keys_t[s] = t->sub[s].n_keys;
    info->n_buckets[s] = t->sub[s].n_buckets;
  }
  info->mean_displacement = t->mean_disp;
  info->max_displacement = t->max_disp;
  info->unique_by_width = (uint32_t)t->classed;
  return EMB_OK;
}

int table_device_bytes(const EmbTable* t, size_t* bytes) {
  if (!t || !bytes) return fail(EMB_EINVAL, "null argument");
  *bytes = t->arena_bytes;
  return EMB_OK;
}

int pass_flash(EmbTable* t, void* d_arena, size_t arena_bytes, emb_stream_t stream) {
  if (!t || !d_arena) return fail(EMB_EINVAL, "null table or arena");
  if (reinterpret_cast<uintptr_t>(d_arena) % 256) return fail(EMB_EINVAL, "arena must be 256-byte aligned");
  if (arena_bytes < t->arena_bytes) return fail(EMB_ENOSPACE, "arena smaller than table_device_bytes()");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (!t->pinned && t->arena_bytes > EmbTable::kBounce && t->ensure_bounce())
    e = flash_bounced(t, static_cast<uint8_t*>(d_arena), t->image, t->arena_bytes, st);
  else
    e = hipMemcpyAsync(d_arena, t->image, t->arena_bytes, hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "pass_flash copy");
  t->d_arena = static_cast<uint8_t*>(d_arena);
  t->flashed = true;
  t->dedup = EmbTable::Dedup{};  // sorted rowrefs of the previous layout are stale
  return EMB_OK;
}

namespace {
bool validate_on() {
  const char* e = std::getenv("EMB_VALIDATE");
  return e && e[0] == '1' && e[1] == 0;
}

// EMB_VALIDATE=1: checks a batch on the device before the call uses it -- offsets start at 0,
// never decrease and end at nnz; with rowrefs, each is a miss or names a whole row of its bag's
// field -- and synchronises the stream to read the verdict.  EMB_EINVAL names what failed.
int validate_batch(EmbTable* t, const int32_t* d_offsets, int64_t n_bags, int64_t nnz,
                   const uint32_t* d_rowref, hipStream_t st, uint32_t* d_flag = nullptr) {
  if (!d_flag && !t->d_vflag) {
    hipError_t e = hipMalloc(reinterpret_cast<void**>(&t->d_vflag), 256);
    if (e != hipSuccess) {
      t->d_vflag = nullptr;
      return hip_fail(e, "EMB_VALIDATE flag allocation");
    }
  }
  ValArgs v{};
  v.d = t->dev();
  v.offsets = d_offsets;
  v.n_bags = (int32_t)n_bags;
  v.nnz = (int32_t)nnz;
  v.rowref = nnz > 0 ? d_rowref : nullptr;
  v.flag = d_flag ? d_flag : t->d_vflag;
  hipError_t e = launch_validate(v, st);
  uint32_t flag = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&flag, v.flag, 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "EMB_VALIDATE check");
  if (flag & 1u) return fail(EMB_EINVAL, "EMB_VALIDATE: offsets[0] is not 0");
  if (flag & 2u) return fail(EMB_EINVAL, "EMB_VALIDATE: offsets decrease");
  if (flag & 4u) return fail(EMB_EINVAL, "EMB_VALIDATE: offsets[n_bags] is not nnz");
  if (flag & 8u)
    return fail(EMB_EINVAL, "EMB_VALIDATE: a rowref is neither a miss nor a row of its bag's field "
                            "inside the table");
  return EMB_OK;
}

// The forward: probe and pool in one launch (mode 0), the probe alone (1) or the pooling of
// earlier rowrefs alone (2).
int forward(EmbTable* t, int mode, const int64_t* d_keys, const int32_t* d_offsets,
            int64_t n_bags, int64_t nnz, void* d_out, int32_t out_dtype, uint32_t* d_rowref,
            int64_t* d_slot, int64_t* d_n_miss, emb_stream_t stream) {
  if (!t) return fail(EMB_EINVAL, "null table");
  if (n_bags < 0 || nnz < 0 || n_bags >= (1ll << 31) || nnz >= (1ll << 31))
    return fail(EMB_EINVAL, "n_bags and nnz must be in [0, 2^31)");
  if (n_bags % t->F) return fail(EMB_EINVAL, "n_bags must be a multiple of n_fields");
  if (mode != 1 && out_dtype != EMB_F32 && out_dtype != EMB_F16) return fail(EMB_EINVAL, "bad out_dtype");
  if (n_bags > 0 && !d_offsets) return fail(EMB_EINVAL, "null offsets");
  if (mode != 1 && n_bags > 0 && !d_out) return fail(EMB_EINVAL, "null output");
  if (nnz > 0 && n_bags == 0) return fail(EMB_EINVAL, "occurrences without bags");
  if (nnz > 0 && !d_rowref) return fail(EMB_EINVAL, "null rowref");
  if (mode != 2 && nnz > 0 && !d_keys) return fail(EMB_EINVAL, "null keys");
  if ((reinterpret_cast<uintptr_t>(d_out) | reinterpret_cast<uintptr_t>(d_rowref)) % 16)
    return fail(EMB_EINVAL, "d_out and d_rowref must be 16-byte aligned");
  if (!t->flashed) return fail(EMB_ESTATE, "lookup before pass_flash");
  if (validate_on() && n_bags > 0) {
    const int rc = validate_batch(t, d_offsets, n_bags, nnz, mode == 2 ? d_rowref : nullptr,
                                  static_cast<hipStream_t>(stream));
    if (rc) return rc;
  }
  FwdLaunch a{};
  a.mode = mode;
  a.d = t->dev();
  a.keys = d_keys;
  a.offsets = d_offsets;
  a.n_bags = (int32_t)n_bags;
  a.nnz = (int32_t)nnz;
  a.out = d_out;
  a.out_f16 = out_dtype == EMB_F16;
  a.rowref = d_rowref;
  a.slot = d_slot;
  a.n_miss = reinterpret_cast<unsigned long long*>(d_n_miss);
  a.probe = (t->flags & EMB_FLAG_PROBE_COOP) ? 1 : (t->flags & EMB_FLAG_PROBE_LANE) ? 2 : 0;
  a.stats = mode == 2 ? nullptr : t->probe_stats;
  LaunchCtx ctx{static_cast<hipStream_t>(stream), &t->timing};
  hipError_t e = launch_lookup_pool(a, ctx);
  if (e != hipSuccess)
    return hip_fail(e, mode == 1 ? "lookup_probe launch" : mode == 2 ? "pool_fwd launch" : "lookup_pool_fwd launch");
  return EMB_OK;
}
}  // namespace

int lookup_pool_fwd(EmbTable* t, const int64_t* d_keys, const int32_t* d_offsets, int64_t n_bags,
                    int64_t nnz, void* d_out, int32_t out_dtype, uint32_t* d_rowref,
                    int64_t* d_slot, int64_t* d_n_miss, emb_stream_t stream) {
  return forward(t, 0, d_keys, d_offsets, n_bags, nnz, d_out, out_dtype, d_rowref, d_slot,
                 d_n_miss, stream);
}

int lookup_probe(EmbTable* t, const int64_t* d_keys, const int32_t* d_offsets, int64_t n_bags,
                 int64_t nnz, uint32_t* d_rowref, int64_t* d_slot, int64_t* d_n_miss,
                 emb_stream_t stream) {
  return forward(t, 1, d_keys, d_offsets, n_bags, nnz, nullptr, EMB_F32, d_rowref, d_slot,
                 d_n_miss, stream);
}

int pool_fwd(EmbTable* t, const uint32_t* d_rowref, const int32_t* d_offsets, int64_t n_bags,
             int64_t nnz, void* d_out, int32_t out_dtype, emb_stream_t stream) {
  return forward(t, 2, nullptr, d_offsets, n_bags, nnz, d_out, out_dtype,
                 const_cast<uint32_t*>(d_rowref), nullptr, nullptr, stream);
}

int table_probe_stats(EmbTable* t, int64_t* d_stats) {
  if (!t) return fail(EMB_EINVAL, "null table");
  if (reinterpret_cast<uintptr_t>(d_stats) % 8) return fail(EMB_EINVAL, "d_stats must be 8-byte aligned");
  t->probe_stats = reinterpret_cast<unsigned long long*>(d_stats);
  return EMB_OK;
}

int bwd_workspace_bytes(const EmbTable* t, int64_t n_bags, int64_t nnz, size_t* bytes) {
  if (!t || !bytes) return fail(EMB_EINVAL, "null argument");
  if (n_bags < 0 || nnz < 0 || nnz >= (1ll << 31)) return fail(EMB_EINVAL, "bad sizes");
  *bytes = plan_bwd(nnz, t->rowref_space, t->max_dim, t->row_dtype == EMB_F16, t->classed).bytes;
  return EMB_OK;
}

namespace {
// The backward shared by both optimizers: dedup, segmented reduction, fused element-wise update.
// stage 0: dedup and update; 1: dedup only (into the workspace); 2: update of a workspace the
// last stage-1 call sorted for the same sizes.
int sparse_bwd(EmbTable* t, int stage, const uint32_t* d_rowref, const int32_t* d_offsets,
               int64_t n_bags, int64_t nnz, const void* d_grad, int32_t grad_dtype, float lr,
               float eps, int ftrl, float beta, float l1, float l2, void* d_ws, size_t ws_bytes,
               uint32_t* d_unique, int32_t* d_count, int64_t* d_n_unique, emb_stream_t stream,
               uint32_t* d_vflag = nullptr) {
  if (!t) return fail(EMB_EINVAL, "null table");
  if (n_bags < 0 || nnz < 0 || n_bags >= (1ll << 31) || nnz >= (1ll << 31))
    return fail(EMB_EINVAL, "n_bags and nnz must be in [0, 2^31)");
  if (n_bags % t->F) return fail(EMB_EINVAL, "n_bags must be a multiple of n_fields");
  if (stage != 1 && grad_dtype != EMB_F32 && grad_dtype != EMB_F16) return fail(EMB_EINVAL, "bad grad_dtype");
  if (nnz > 0 && n_bags == 0) return fail(EMB_EINVAL, "occurrences without bags");
  if (nnz > 0 && stage != 2 && (!d_rowref || !d_offsets))
    return fail(EMB_EINVAL, "null rowref or offsets");
  if (nnz > 0 && stage != 1 && !d_grad) return fail(EMB_EINVAL, "null grad");
  if (nnz > 0 && !d_ws) return fail(EMB_EINVAL, "null workspace");
  if (d_count && !d_unique) return fail(EMB_EINVAL, "d_count needs d_unique");
  if ((reinterpret_cast<uintptr_t>(d_grad) | reinterpret_cast<uintptr_t>(d_rowref) |
       reinterpret_cast<uintptr_t>(d_ws)) % 16)
    return fail(EMB_EINVAL, "d_grad, d_rowref and d_ws must be 16-byte aligned");
  if (ftrl && !(lr > 0.f && beta >= 0.f && l1 >= 0.f && l2 >= 0.f && std::isfinite(lr) &&
                std::isfinite(beta) && std::isfinite(l1) && std::isfinite(l2)))
    return fail(EMB_EINVAL, "FTRL needs alpha > 0 and finite beta, l1, l2 >= 0");
  const BwdPlan p = plan_bwd(nnz, t->rowref_space, t->max_dim, t->row_dtype == EMB_F16, t->classed);
  if (nnz > 0 && ws_bytes < p.bytes) return fail(EMB_ENOSPACE, "workspace smaller than bwd_workspace_bytes()");
  if (ftrl && !t->ftrl) return fail(EMB_ESTATE, "table keeps no FTRL state (EMB_FLAG_FTRL)");
  if (!t->flashed) return fail(EMB_ESTATE, "backward before pass_flash");
  if (stage == 2 && (t->dedup.ws != d_ws || t->dedup.nnz != nnz || t->dedup.n_bags != n_bags))
    return fail(EMB_ESTATE, "apply without a sparse_bwd_dedup of this workspace and these sizes");
  if (stage != 2 && validate_on() && n_bags > 0) {
    const int rc = validate_batch(t, d_offsets, n_bags, nnz, d_rowref,
                                  static_cast<hipStream_t>(stream), d_vflag);
    if (rc) return rc;
  }
  // a dedup enables one apply; any other backward call may overwrite its workspace
  t->dedup = EmbTable::Dedup{};
  BwdLaunch a{};
  a.stage = stage;
  a.d = t->dev();
  a.rowref = d_rowref;
  a.offsets = d_offsets;
  a.n_bags = (int32_t)n_bags;
  a.nnz = (int32_t)nnz;
  a.grad = d_grad;
  a.grad_f16 = grad_dtype == EMB_F16;
  a.lr = lr;
  a.eps = eps;
  a.ftrl = ftrl;
  a.beta = beta;
  a.l1 = l1;
  a.l2 = l2;
  a.ws = d_ws;
  a.ws_bytes = ws_bytes;
  a.unique = d_unique;
  a.count = d_count;
  a.n_unique = d_n_unique;
  LaunchCtx ctx{static_cast<hipStream_t>(stream), &t->timing};
  hipError_t e = launch_sparse_bwd(a, p, ctx);
  if (e != hipSuccess)
    return hip_fail(e, stage == 1 ? "sparse_bwd_dedup launch"
                       : ftrl ? "sparse_ftrl_bwd launch" : "sparse_adagrad_bwd launch");
  if (stage == 1) {
    t->dedup.ws = d_ws;
    t->dedup.nnz = nnz;
    t->dedup.n_bags = n_bags;
  }
  return EMB_OK;
}
}  // namespace

int sparse_bwd_dedup(EmbTable* t, const uint32_t* d_rowref, const int32_t* d_offsets,
                     int64_t n_bags, int64_t nnz, void* d_ws, size_t ws_bytes,
                     emb_stream_t stream) {
  return sparse_bwd(t, 1, d_rowref, d_offsets, n_bags, nnz, nullptr, EMB_F32, 0.f, 0.f, 0, 0.f,
                    0.f, 0.f, d_ws, ws_bytes, nullptr, nullptr, nullptr, stream);
}

int sparse_adagrad_apply(EmbTable* t, int64_t n_bags, int64_t nnz, const void* d_grad,
                         int32_t grad_dtype, float lr, float eps, void* d_ws, size_t ws_bytes,
                         uint32_t* d_unique, int32_t* d_count, int64_t* d_n_unique,
                         emb_stream_t stream) {
  return sparse_bwd(t, 2, nullptr, nullptr, n_bags, nnz, d_grad, grad_dtype, lr, eps, 0, 0.f,
                    0.f, 0.f, d_ws, ws_bytes, d_unique, d_count, d_n_unique, stream);
}

int sparse_ftrl_apply(EmbTable* t, int64_t n_bags, int64_t nnz, const void* d_grad,
                      int32_t grad_dtype, float alpha, float beta, float l1, float l2, void* d_ws,
                      size_t ws_bytes, uint32_t* d_unique, int32_t* d_count,
                      int64_t* d_n_unique, emb_stream_t stream) {
  return sparse_bwd(t, 2, nullptr, nullptr, n_bags, nnz, d_grad, grad_dtype, alpha, 0.f, 1, beta,
                    l1, l2, d_ws, ws_bytes, d_unique, d_count, d_n_unique, stream);
}

int sparse_adagrad_bwd(EmbTable* t, const uint32_t* d_rowref, const int32_t* d_offsets,
                       int64_t n_bags, int64_t nnz, const void* d_grad, int32_t grad_dtype,
                       float lr, float eps, void* d_ws, size_t ws_bytes, uint32_t* d_unique,
                       int32_t* d_count, int64_t* d_n_unique, emb_stream_t stream) {
  return sparse_bwd(t, 0, d_rowref, d_offsets, n_bags, nnz, d_grad, grad_dtype, lr, eps, 0, 0.f,
                    0.f, 0.f, d_ws, ws_bytes, d_unique, d_count, d_n_unique, stream);
}

int sparse_adagrad_bwd_noalloc(EmbTable* t, const uint32_t* d_rowref, const int32_t* d_offsets,
                               int64_t n_bags, int64_t nnz, const void* d_grad, int32_t grad_dtype,
                               float lr, float eps, uint32_t* d_unique, int32_t* d_count,
                               int64_t* d_n_unique, emb_stream_t stream) {
  if (!t) return fail(EMB_EINVAL, "null table");
  if (n_bags < 0 || nnz < 0 || nnz >= (1ll << 31)) return fail(EMB_EINVAL, "bad sizes");
  // the scratch holds the workspace and, at its end, the EMB_VALIDATE flag word
  const size_t need = plan_bwd(nnz, t->rowref_space, t->max_dim, t->row_dtype == EMB_F16,
                               t->classed).bytes;
  const size_t cap = scratch_bytes() - 256;
  if (need > cap)
    return fail(EMB_ENOSPACE, "batch needs " + std::to_string(need) + " bytes of backward "
                              "workspace; the static scratch holds " + std::to_string(cap));
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return hip_fail(e, "static scratch address");
  uint32_t* vflag = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + cap);
  return sparse_bwd(t, 0, d_rowref, d_offsets, n_bags, nnz, d_grad, grad_dtype, lr, eps, 0, 0.f,
                    0.f, 0.f, ws, cap, d_unique, d_count, d_n_unique, stream, vflag);
}

int sparse_ftrl_bwd(EmbTable* t, const uint32_t* d_rowref, const int32_t* d_offsets,
                    int64_t n_bags, int64_t nnz, const void* d_grad, int32_t grad_dtype,
                    float alpha, float beta, float l1, float l2, void* d_ws, size_t ws_bytes,
                    uint32_t* d_unique, int32_t* d_count, int64_t* d_n_unique,
                    emb_stream_t stream) {
  return sparse_bwd(t, 0, d_rowref, d_offsets, n_bags, nnz, d_grad, grad_dtype, alpha, 0.f, 1,
                    beta, l1, l2, d_ws, ws_bytes, d_unique, d_count, d_n_unique, stream);
}

int pass_writeback(EmbTable* t, emb_stream_t stream) {
  if (!t) return fail(EMB_EINVAL, "null table");
  if (!t->flashed) return fail(EMB_ESTATE, "write-back before pass_flash");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t n = t->off_meta - t->off_rows;
  hipError_t e;
  if (!t->pinned && n > EmbTable::kBounce && t->ensure_bounce())
    e = writeback_bounced(t, t->image + t->off_rows, t->d_arena + t->off_rows, n, s);
  else
    e = hipMemcpyAsync(t->image + t->off_rows, t->d_arena + t->off_rows, n,
                       hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "pass_writeback copy");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "pass_writeback sync");
  return EMB_OK;
}

namespace {
// Bytes one rowref unit takes in the compacted write-back: its index, row elements, accumulator
// and master.
size_t wb_unit_bytes(const EmbTable* t) {
  const size_t g = (size_t)t->granule;
  return 4 + g * t->elem_bytes + 4 * g + (t->has_master ? 4 * g : 0) + (t->ftrl ? 4 * g : 0);
}
size_t wb_blocks(const EmbTable* t) { return (t->touched_words + kWbWords - 1) / kWbWords; }
size_t wb_head_bytes(const EmbTable* t) { return align256(4 * (wb_blocks(t) + 1)); }
// one half of the workspace holds at least one bitmap block's worth of units
size_t wb_min_half(const EmbTable* t) { return align256((size_t)kWbWords * 32 * wb_unit_bytes(t) + 16); }

// Compacted piece of n units: unit indices, then rows, accumulators, masters (16-byte aligned).
struct WbPiece {
  size_t rows, acc, master, linear, bytes;
};
WbPiece wb_piece(const EmbTable* t, size_t n) {
  const size_t g = (size_t)t->granule;
  WbPiece p;
  p.rows = (4 * n + 15) & ~(size_t)15;
  p.acc = p.rows + n * g * t->elem_bytes;
  p.master = p.acc + n * g * 4;
  p.linear = p.master + (t->has_master ? n * g * 4 : 0);
  p.bytes = p.linear + (t->ftrl ? n * g * 4 : 0);
  return p;
}

// Host side of one piece: each unit's row, accumulator and master into the image (runs of
// consecutive units in one copy), and their dirty bits.
void wb_scatter(EmbTable* t, const uint8_t* h, size_t n) {
  const WbPiece p = wb_piece(t, n);
  const size_t g = (size_t)t->granule, rb = g * t->elem_bytes;
  const uint32_t* u = reinterpret_cast<const uint32_t*>(h);
  uint8_t* R = t->image + t->off_rows;
  uint8_t* A = t->image + t->off_acc;
  uint8_t* M = t->image + t->off_master;
  uint8_t* L = t->image + t->off_linear;
  parallel_for(n, [&](size_t b, size_t e) {
    for (size_t i = b; i < e;) {
      size_t j = i + 1;
      while (j < e && u[j] == u[j - 1] + 1) ++j;
      const size_t len = j - i, u0 = u[i];
      std::memcpy(R + u0 * rb, h + p.rows + i * rb, len * rb);
      std::memcpy(A + u0 * g * 4, h + p.acc + i * g * 4, len * g * 4);
      if (t->has_master) std::memcpy(M + u0 * g * 4, h + p.master + i * g * 4, len * g * 4);
      if (t->ftrl) std::memcpy(L + u0 * g * 4, h + p.linear + i * g * 4, len * g * 4);
      for (; i < j; ++i) __atomic_fetch_or(&t->dirty[u[i] >> 6], 1ull << (u[i] & 63), __ATOMIC_RELAXED);
    }
  });
}
}  // namespace

int writeback_workspace_bytes(const EmbTable* t, size_t* min_bytes) {
  if (!t || !min_bytes) return fail(EMB_EINVAL, "null argument");
  if (!(t->flags & EMB_FLAG_TRACK_TOUCHED)) return fail(EMB_ESTATE, "table does not track touched rows");
  *min_bytes = wb_head_bytes(t) + 2 * wb_min_half(t);
  return EMB_OK;
}

int pass_writeback_touched(EmbTable* t, void* d_ws, size_t ws_bytes, int64_t* n_units_out,
                           emb_stream_t stream) {
  if (!t) return fail(EMB_EINVAL, "null table");
  if (!(t->flags & EMB_FLAG_TRACK_TOUCHED)) return fail(EMB_ESTATE, "table does not track touched rows");
  if (!t->flashed) return fail(EMB_ESTATE, "write-back before pass_flash");
  if (!d_ws || reinterpret_cast<uintptr_t>(d_ws) % 256) return fail(EMB_EINVAL, "workspace must be 256-byte aligned");
  const size_t head = wb_head_bytes(t);
  if (ws_bytes < head + 2 * wb_min_half(t)) return fail(EMB_ENOSPACE, "workspace smaller than writeback_workspace_bytes()");
  t->dedup = EmbTable::Dedup{};  // the workspace may be a deduplicated backward's: it is overwritten
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t ub = wb_unit_bytes(t);
  const bool pin = t->ensure_bounce();
  std::vector<uint8_t> pageable[2];
  const size_t half = ((ws_bytes - head) / 2) & ~(size_t)255;
  const size_t host_cap = pin ? EmbTable::kBounce : half;
  // units one piece may hold: bounded by a workspace half and a host buffer
  const size_t cap = (std::min(half, host_cap) - 16) / ub;
  uint8_t* ws = static_cast<uint8_t*>(d_ws);

  WbLaunch a{};
  a.touched = t->dev().touched;
  a.n_words = (int64_t)t->touched_words;
  a.granule = t->granule;
  a.row_bytes = (int32_t)(t->granule * t->elem_bytes);
  a.has_master = t->has_master;
  a.rows = t->d_arena + t->off_rows;
  a.acc = reinterpret_cast<const float*>(t->d_arena + t->off_acc);
  a.master = t->has_master ? reinterpret_cast<const float*>(t->d_arena + t->off_master) : nullptr;
  a.linear = t->ftrl ? reinterpret_cast<const float*>(t->d_arena + t->off_linear) : nullptr;
  a.bcount = reinterpret_cast<uint32_t*>(ws);
  a.blocks = (int64_t)wb_blocks(t);
  std::vector<uint32_t> pre((size_t)a.blocks + 1, 0);
  hipError_t e = launch_wb_count(a, st);
  if (e == hipSuccess) e = launch_wb_scan(a, st);
  if (e == hipSuccess && a.blocks > 0)
    e = hipMemcpyAsync(pre.data(), a.bcount, 4 * pre.size(), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "pass_writeback_touched count");
  if (t->dirty.empty()) t->dirty.assign(((size_t)t->rowref_space + 63) / 64, 0);

  // pieces: runs of whole bitmap blocks whose units fit one piece
  std::vector<std::pair<int64_t, int64_t>> pieces;
  for (int64_t b0 = 0; b0 < a.blocks;) {
    int64_t b1 = b0 + 1;
    while (b1 < a.blocks && (size_t)(pre[(size_t)b1 + 1] - pre[(size_t)b0]) <= cap) ++b1;
    if (pre[(size_t)b1] > pre[(size_t)b0]) pieces.emplace_back(b0, b1);
    b0 = b1;
  }
  auto count = [&](size_t k) { return (size_t)(pre[(size_t)pieces[k].second] - pre[(size_t)pieces[k].first]); };
  auto host_buf = [&](int b) -> uint8_t* {
    if (pin) return t->bounce[b];
    if (pageable[b].empty()) pageable[b].resize(half);
    return pageable[b].data();
  };
  // piece k: compact into workspace half k % 2, copy into host buffer k % 2
  auto issue = [&](size_t k) {
    const int b = (int)(k & 1);
    const size_t n = count(k);
    const WbPiece p = wb_piece(t, n);
    uint8_t* o = ws + head + (size_t)b * half;
    WbLaunch g = a;
    g.b0 = pieces[k].first;
    g.b1 = pieces[k].second;
    g.base = pre[(size_t)g.b0];
    g.out_unit = reinterpret_cast<uint32_t*>(o);
    g.out_rows = o + p.rows;
    g.out_acc = reinterpret_cast<float*>(o + p.acc);
    g.out_master = reinterpret_cast<float*>(o + p.master);
    g.out_linear = reinterpret_cast<float*>(o + p.linear);
    hipError_t r = launch_wb_gather(g, st);
    if (r == hipSuccess) r = hipMemcpyAsync(host_buf(b), o, p.bytes, hipMemcpyDeviceToHost, st);
    if (r == hipSuccess) r = pin ? hipEventRecord(t->bounce_ev[b], st) : hipStreamSynchronize(st);
    return r;
  };
  if (!pieces.empty()) e = issue(0);
  for (size_t k = 0; k < pieces.size() && e == hipSuccess; ++k) {
    if (k + 1 < pieces.size()) e = issue(k + 1);
    const int b = (int)(k & 1);
    if (e == hipSuccess && pin) e = hipEventSynchronize(t->bounce_ev[b]);
    if (e != hipSuccess) break;
    wb_scatter(t, host_buf(b), count(k));
  }
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "pass_writeback_touched copy");
  if (n_units_out) *n_units_out = a.blocks > 0 ? (int64_t)pre[(size_t)a.blocks] : 0;
  return EMB_OK;
}

int table_dirty_keys(EmbTable* t, int64_t* keys_out, int64_t cap, int64_t* n_out, int clear) {
  if (!t || !n_out || cap < 0) return fail(EMB_EINVAL, "null argument or negative capacity");
  int64_t n = 0;
  if (!t->dirty.empty()) {
    for (size_t r = 0; r < t->row_ref.size(); ++r) {
      const uint32_t u = t->row_ref[r];
      if (!((t->dirty[u >> 6] >> (u & 63)) & 1ull)) continue;
      if (keys_out && n < cap) keys_out[n] = (int64_t)t->row_keys[r];
      ++n;
    }
  }
  *n_out = n;
  if (keys_out && n > cap) return fail(EMB_ENOSPACE, "table_dirty_keys: more dirty keys than cap");
  if (clear) std::fill(t->dirty.begin(), t->dirty.end(), 0ull);
  return EMB_OK;
}

int table_carry_state(EmbTable* dst, const EmbTable* src, int64_t* n_carried) {
  if (!dst || !src) return fail(EMB_EINVAL, "null table");
  if (dst->F != src->F || dst->dim != src->dim || dst->row_dtype != src->row_dtype ||
      dst->has_master != src->has_master || dst->ftrl != src->ftrl)
    return fail(EMB_EINVAL, "table_carry_state: tables differ in fields, dims, row dtype, master or FTRL state");
  const size_t eb = dst->elem_bytes;
  std::atomic<int64_t> carried{0};
  parallel_for(dst->row_keys.size(), [&](size_t b, size_t e) {
    int64_t c = 0;
    for (size_t r = b; r < e; ++r) {
      const uint64_t k = dst->row_keys[r];
      uint32_t rr;
      int64_t sl;
      if (!src->probe(k, &rr, &sl)) continue;
      const uint64_t D = (uint64_t)dst->dim[(int)(k >> 48)];
      const uint64_t s0 = (uint64_t)rr * (uint64_t)src->granule;
      const uint64_t d0 = (uint64_t)dst->row_ref[r] * (uint64_t)dst->granule;
      std::memcpy(dst->image + dst->off_rows + d0 * eb, src->image + src->off_rows + s0 * eb, D * eb);
      std::memcpy(dst->image + dst->off_acc + d0 * 4, src->image + src->off_acc + s0 * 4, D * 4);
      if (dst->has_master)
        std::memcpy(dst->image + dst->off_master + d0 * 4, src->image + src->off_master + s0 * 4, D * 4);
      if (dst->ftrl)
        std::memcpy(dst->image + dst->off_linear + d0 * 4, src->image + src->off_linear + s0 * 4, D * 4);
      ++c;
    }
    carried += c;
  });
  if (n_carried) *n_carried = carried.load();
  return EMB_OK;
}

int table_export(const EmbTable* t, const int64_t* keys, int64_t n, void* rows, float* acc,
                 float* master) {
  if (!t || (n > 0 && !keys)) return fail(EMB_EINVAL, "null argument");
  if (master && !t->has_master) return fail(EMB_EINVAL, "table keeps no master copy");
  const size_t eb = t->elem_bytes;
  uint64_t o = 0;
  for (int64_t i = 0; i < n; ++i) {
    uint32_t rr;
    int64_t sl;
    const uint64_t k = (uint64_t)keys[i];
    if (!t->probe(k, &rr, &sl)) return fail(EMB_EINVAL, "table_export: key not in the table");
    const uint64_t D = (uint64_t)t->dim[(int)(k >> 48)];
    const uint64_t e = (uint64_t)rr * (uint64_t)t->granule;
    if (rows) std::memcpy(static_cast<uint8_t*>(rows) + o * eb, t->image + t->off_rows + e * eb, D * eb);
    if (acc) std::memcpy(acc + o, reinterpret_cast<const float*>(t->image + t->off_acc) + e, D * 4);
    if (master) std::memcpy(master + o, reinterpret_cast<const float*>(t->image + t->off_master) + e, D * 4);
    o += D;
  }
  return EMB_OK;
}

int table_fill_state(EmbTable* t, int64_t first, int64_t n, const void* rows, const float* acc,
                     const float* master) {
  if (!t) return fail(EMB_EINVAL, "null table");
  if (first < 0 || n < 0 || (uint64_t)first + (uint64_t)n > t->n_keys)
    return fail(EMB_EINVAL, "table_fill_state: key range outside the key list given at create");
  if (master && !t->has_master) return fail(EMB_EINVAL, "table keeps no master copy");
  if (n == 0 || (!rows && !acc && !master)) return EMB_OK;
  const size_t eb = t->elem_bytes;
  const bool f16 = t->row_dtype == EMB_F16;
  // element offset of each key's slice inside the caller's packed arrays
  std::vector<uint64_t> off;
  if (t->var_dim) {
    off.resize((size_t)n + 1, 0);
    for (int64_t i = 0; i < n; ++i) {
      const uint64_t k = t->row_keys[t->row_of_key[(size_t)(first + i)]];
      off[(size_t)i + 1] = off[(size_t)i] + (uint64_t)t->dim[(int)(k >> 48)];
    }
  }
  uint8_t* R = t->image + t->off_rows;
  float* A = reinterpret_cast<float*>(t->image + t->off_acc);
  float* M = t->has_master ? reinterpret_cast<float*>(t->image + t->off_master) : nullptr;
  parallel_for((size_t)n, [&](size_t b, size_t e) {
    for (size_t i = b; i < e; ++i) {
      const uint32_t r = t->row_of_key[(size_t)first + i];
      const uint64_t D = (uint64_t)t->dim[(int)(t->row_keys[r] >> 48)];
      const uint64_t src = t->var_dim ? off[i] : (uint64_t)i * D;
      const uint64_t dst = (uint64_t)t->row_ref[r] * (uint64_t)t->granule;
      if (rows) {
        std::memcpy(R + dst * eb, static_cast<const uint8_t*>(rows) + src * eb, D * eb);
      } else if (master && f16) {
        uint16_t* h = reinterpret_cast<uint16_t*>(R) + dst;
        for (uint64_t q = 0; q < D; ++q) h[q] = f32_to_f16(master[src + q]);
      }
      if (acc) std::memcpy(A + dst, acc + src, D * 4);
      if (M) {
        if (master) {
          std::memcpy(M + dst, master + src, D * 4);
        } else if (rows) {
          const uint16_t* h = reinterpret_cast<const uint16_t*>(R) + dst;
          for (uint64_t q = 0; q < D; ++q) M[dst + q] = f16_to_f32(h[q]);
        }
      }
    }
  });
  return EMB_OK;
}

int table_fill_linear(EmbTable* t, int64_t first, int64_t n, const float* z) {
  if (!t) return fail(EMB_EINVAL, "null table");
  if (!t->ftrl) return fail(EMB_EINVAL, "table keeps no FTRL state (EMB_FLAG_FTRL)");
  if (first < 0 || n < 0 || (uint64_t)first + (uint64_t)n > t->n_keys)
    return fail(EMB_EINVAL, "table_fill_linear: key range outside the key list given at create");
  if (n == 0) return EMB_OK;
  if (!z) return fail(EMB_EINVAL, "null linear state");
  std::vector<uint64_t> off;
  if (t->var_dim) {
    off.resize((size_t)n + 1, 0);
    for (int64_t i = 0; i < n; ++i) {
      const uint64_t k = t->row_keys[t->row_of_key[(size_t)(first + i)]];
      off[(size_t)i + 1] = off[(size_t)i] + (uint64_t)t->dim[(int)(k >> 48)];
    }
  }
  float* L = reinterpret_cast<float*>(t->image + t->off_linear);
  parallel_for((size_t)n, [&](size_t b, size_t e) {
    for (size_t i = b; i < e; ++i) {
      const uint32_t r = t->row_of_key[(size_t)first + i];
      const uint64_t D = (uint64_t)t->dim[(int)(t->row_keys[r] >> 48)];
      const uint64_t src = t->var_dim ? off[i] : (uint64_t)i * D;
      std::memcpy(L + (uint64_t)t->row_ref[r] * (uint64_t)t->granule, z + src, D * 4);
    }
  });
  return EMB_OK;
}

int table_export_linear(const EmbTable* t, const int64_t* keys, int64_t n, float* z) {
  if (!t || (n > 0 && (!keys || !z))) return fail(EMB_EINVAL, "null argument");
  if (!t->ftrl) return fail(EMB_EINVAL, "table keeps no FTRL state (EMB_FLAG_FTRL)");
  const float* L = reinterpret_cast<const float*>(t->image + t->off_linear);
  uint64_t o = 0;
  for (int64_t i = 0; i < n; ++i) {
    uint32_t rr;
    int64_t sl;
    const uint64_t k = (uint64_t)keys[i];
    if (!t->probe(k, &rr, &sl)) return fail(EMB_EINVAL, "table_export_linear: key not in the table");
    const uint64_t D = (uint64_t)t->dim[(int)(k >> 48)];
    std::memcpy(z + o, L + (uint64_t)rr * (uint64_t)t->granule, D * 4);
    o += D;
  }
  return EMB_OK;
}

int table_key_rowref(const EmbTable* t, const int64_t* keys, int64_t n, uint32_t* rowref,
                     int64_t* slot) {
  if (!t || (n > 0 && (!keys || !rowref))) return fail(EMB_EINVAL, "null argument");
  parallel_for((size_t)n, [&](size_t b, size_t e) {
    for (size_t i = b; i < e; ++i) {
      uint32_t rr = kMiss;
      int64_t sl = -1;
      if (!t->probe((uint64_t)keys[i], &rr, &sl)) { rr = kMiss; sl = -1; }
      rowref[i] = rr;
      if (slot) slot[i] = sl;
    }
  });
  return EMB_OK;
}

int table_rowref_keys(const EmbTable* t, const uint32_t* rowrefs, int64_t n, int64_t* keys_out) {
  if (!t || (n > 0 && (!rowrefs || !keys_out))) return fail(EMB_EINVAL, "null argument");
  for (int64_t i = 0; i < n; ++i) {
    auto it = std::lower_bound(t->row_ref.begin(), t->row_ref.end(), rowrefs[i]);
    if (it == t->row_ref.end() || *it != rowrefs[i])
      return fail(EMB_EINVAL, "table_rowref_keys: not a row start");
    keys_out[i] = (int64_t)t->row_keys[(size_t)(it - t->row_ref.begin())];
  }
  return EMB_OK;
}

int emb_timing_enable(EmbTable* t, int enable, const char* only) {
  if (!t) return fail(EMB_EINVAL, "null table");
  t->timing.on = enable != 0;
  t->timing.only = only ? only : "";
  t->timing.used = 0;
  return EMB_OK;
}

int emb_timing_read(EmbTable* t, char* names, size_t name_cap, int64_t* counts, double* ms,
                    int32_t cap, int32_t* n_out) {
  if (!t || !n_out) return fail(EMB_EINVAL, "null argument");
  Timing& T = t->timing;
  std::vector<std::string> nm;
  std::vector<int64_t> cnt;
  std::vector<double> tot;
  for (size_t i = 0; i < T.used; ++i) {
    Timing::Rec& r = T.pool[i];
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return hip_fail(e, "timing event sync");
    float x = 0.f;
    e = hipEventElapsedTime(&x, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e, "timing elapsed");
    size_t k = 0;
    while (k < nm.size() && nm[k] != r.name) ++k;
    if (k == nm.size()) { nm.push_back(r.name); cnt.push_back(0); tot.push_back(0.0); }
    cnt[k] += 1;
    tot[k] += x;
  }
  T.used = 0;
  std::string joined;
  for (size_t k = 0; k < nm.size(); ++k) joined += nm[k] + "\n";
  if (names && name_cap) {
    const size_t c = std::min(name_cap - 1, joined.size());
    std::memcpy(names, joined.data(), c);
    names[c] = 0;
  }
  const int32_t m = (int32_t)std::min<size_t>(nm.size(), (size_t)(cap > 0 ? cap : 0));
  for (int32_t k = 0; k < m; ++k) {
    if (counts) counts[k] = cnt[k];
    if (ms) ms[k] = tot[k];
  }
  *n_out = (int32_t)nm.size();
  return EMB_OK;
}

void table_destroy(EmbTable* t) { delete t; }

}  // extern "C"
