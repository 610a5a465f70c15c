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

#include "emb_internal.h"

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

// ---------------------------------------------------------------- wave / block helpers
__device__ __forceinline__ int lane_id() { return __lane_id(); }

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
struct TabSel {
  const uint64_t* buckets;
  uint32_t n_home, n_buckets;
};
__device__ __forceinline__ TabSel pick_tab(const DevDesc& d, uint64_t key) {
  const bool one = (d.n_tables == 2) && (key & 1ull);
  TabSel s;
  s.buckets = one ? d.tab[1].buckets : d.tab[0].buckets;
  s.n_home = one ? d.tab[1].n_home : d.tab[0].n_home;
  s.n_buckets = one ? d.tab[1].n_buckets : d.tab[0].n_buckets;
  return s;
}

// Ordered linear probing over 128-byte buckets of 15 keys: scan from the home slot until the key
// or an empty slot.  On a hit the rowref is the bucket's stored prefix plus the row units of the
// occupied slots before the hit (rows are stored in slot order).
__device__ __forceinline__ uint32_t probe_key(const DevDesc& d, uint64_t key, int bag_field,
                                              int64_t& slot) {
  slot = -1;
  if (key == kEmpty || (int)(key >> 48) != bag_field) return kMiss;
  const TabSel tb = pick_tab(d, key);
  const uint32_t home = home_slot(mix64(key), tb.n_home);
  uint32_t b = home / (uint32_t)kKeysPerBucket;
  uint32_t l0 = home - b * (uint32_t)kKeysPerBucket;
  for (;;) {
    if (b >= tb.n_buckets) return kMiss;  // unreachable with a well-formed terminator bucket
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
      if (!d.var_dim) {
        rr += __builtin_popcount(below);
      } else {
#pragma unroll
        for (int q = 0; q < kKeysPerBucket; ++q) {
          const uint64_t w = (q & 1) ? v[q >> 1].y : v[q >> 1].x;
          if ((below >> q) & 1u) rr += (uint32_t)d.fgran[(int)(w >> 48)];
        }
      }
      slot = (int64_t)b * kKeysPerBucket + l;
      return rr;
    }
    ++b;
    l0 = 0;
  }
}

// ---------------------------------------------------------------- forward: probe + sum pool
constexpr int kFwdBags = 256;    // bags per block
constexpr int kFwdKeyCap = 4096; // rowrefs staged in LDS; larger blocks re-read them from HBM/L2

template <typename RowT, typename OutT>
__global__ __launch_bounds__(kBlock) void k_lookup_pool(FwdLaunch a, int gs_log2) {
  constexpr int EPL = 16 / (int)sizeof(RowT);  // row elements per lane: one 16-byte load
  typedef typename F32V<EPL>::t AccV;
  __shared__ int32_t s_off[kFwdBags + 1];
  __shared__ uint32_t s_rr[kFwdKeyCap];
  __shared__ uint32_t s_miss;
  const int tid = threadIdx.x;
  const int32_t j0 = (int32_t)blockIdx.x * kFwdBags;
  const int nb = min(kFwdBags, a.n_bags - j0);
  // offsets are clamped into [0, nnz] so malformed input cannot reach outside the buffers
  for (int i = tid; i <= nb; i += kBlock) s_off[i] = min(max(a.offsets[j0 + i], 0), a.nnz);
  if (tid == 0) s_miss = 0;
  __syncthreads();
  const int32_t base = s_off[0];
  const int32_t nk = max(s_off[nb] - base, 0);
  const bool in_lds = nk <= kFwdKeyCap;
  const int F = a.d.n_fields;
  const int f0 = j0 % F;

  // phase 1: one lane per key
  uint32_t miss = 0;
  for (int i = tid; i < nk; i += kBlock) {
    const int32_t pos = base + i;
    const uint64_t key = (uint64_t)a.keys[pos];
    int lo = 0, hi = nb - 1;  // last bag whose start is <= pos
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= pos) lo = mid; else hi = mid - 1;
    }
    int64_t sl;
    const uint32_t rr = probe_key(a.d, key, (f0 + lo) % F, sl);
    miss += (rr == kMiss);
    if (in_lds) s_rr[i] = rr;
    a.rowref[pos] = rr;
    if (a.slot) a.slot[pos] = sl;
  }
  if (miss) atomicAdd(&s_miss, miss);
  __syncthreads();
  if (tid == 0 && s_miss && a.n_miss) atomicAdd(a.n_miss, (unsigned long long)s_miss);

  // phase 2: a group of 2^gs_log2 lanes per bag, EPL elements per lane
  const int lane = tid & ((1 << gs_log2) - 1);
  const int ngrp = kBlock >> gs_log2;
  const RowT* rows = reinterpret_cast<const RowT*>(a.d.rows);
  OutT* out = reinterpret_cast<OutT*>(a.out);
  for (int jb = tid >> gs_log2; jb < nb; jb += ngrp) {
    const int f = (f0 + jb) % F;
    const int D = a.d.var_dim ? a.d.fdim[f] : a.d.fixed_dim;
    const int col = a.d.var_dim ? a.d.fcol[f] : f * a.d.fixed_dim;
    const int e0 = lane * EPL;
    if (e0 >= D) continue;
    const int32_t b = (j0 + jb) / F;
    const int k0 = min(max(s_off[jb] - base, 0), nk), k1 = min(max(s_off[jb + 1] - base, k0), nk);
    AccV acc = 0.0f;
    int k = k0;
    for (; k + 4 <= k1; k += 4) {
      uint32_t r[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) r[u] = in_lds ? s_rr[k + u] : a.rowref[base + k + u];
      AccV x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        x[u] = (r[u] != kMiss)
                   ? load_f32<RowT, EPL>(rows + (uint64_t)r[u] * a.d.granule + e0)
                   : AccV(0.0f);
#pragma unroll
      for (int u = 0; u < 4; ++u) acc += x[u];
    }
    for (; k < k1; ++k) {
      const uint32_t r = in_lds ? s_rr[k] : a.rowref[base + k];
      if (r != kMiss) acc += load_f32<RowT, EPL>(rows + (uint64_t)r * a.d.granule + e0);
    }
    store_from_f32<OutT, EPL>(out + (uint64_t)b * a.d.out_width + col + e0, acc);
  }
}

// ---------------------------------------------------------------- backward: radix sort
constexpr int kIPT = 8;                       // items per thread per sort tile
constexpr int kTile = kBlock * kIPT;          // 2048
constexpr int kOffStage = 2048;               // bag offsets staged in LDS for the first pass
constexpr int kQ = 16;                        // sorted items scanned per lane group (update pass)
constexpr int kLong = 32;                     // segments longer than this take the block path

struct SortArgs {
  const uint32_t* rowref;   // first pass source
  const int32_t* offsets;
  int32_t n_bags;
  const uint32_t* kin;
  const uint32_t* vin;
  uint32_t* kout;
  uint32_t* vout;
  uint32_t* counts;   // [256][tiles]
  uint32_t* tot;      // [256]
  uint32_t* ctr;      // small counters, zeroed by the first scan
  int32_t n;
  int32_t tiles;
  uint32_t miss_key;
  int32_t shift;
};

// Sort key of an occurrence: its rowref, or miss_key (= rowref space, sorts last) for a miss or any
// value outside the table.
__device__ __forceinline__ uint32_t first_key(uint32_t rr, uint32_t miss_key) {
  return rr >= miss_key ? miss_key : rr;
}

// Per-tile histogram of one 8-bit digit.
template <bool FIRST>
__global__ __launch_bounds__(kBlock) void k_sort_hist(SortArgs a) {
  __shared__ uint32_t h[256];
  const int t = blockIdx.x;
  h[threadIdx.x] = 0;
  __syncthreads();
  const int32_t i0 = t * kTile;
  const int32_t i1 = min(a.n, i0 + kTile);
  for (int32_t i = i0 + threadIdx.x; i < i1; i += kBlock) {
    const uint32_t k = FIRST ? first_key(a.rowref[i], a.miss_key) : a.kin[i];
    atomicAdd(&h[(k >> a.shift) & 255u], 1u);
  }
  __syncthreads();
  a.counts[(size_t)threadIdx.x * a.tiles + t] = h[threadIdx.x];
}

// Exclusive scan of each digit's per-tile counts (one block per digit) and the digit totals.
__global__ __launch_bounds__(kBlock) void k_sort_scan(SortArgs a, int zero_ctr) {
  __shared__ uint32_t s_w[kWaves];
  const int d = blockIdx.x;
  if (zero_ctr && d == 0 && threadIdx.x < 16) a.ctr[threadIdx.x] = 0;
  uint32_t* row = a.counts + (size_t)d * a.tiles;
  uint32_t carry = 0;
  for (int32_t c0 = 0; c0 < a.tiles; c0 += kBlock * 4) {
    uint32_t v[4], s = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int32_t i = c0 + threadIdx.x * 4 + u;
      v[u] = i < a.tiles ? row[i] : 0u;
      s += v[u];
    }
    uint32_t total;
    uint32_t pre = block_excl_scan(s, s_w, total) + carry;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int32_t i = c0 + threadIdx.x * 4 + u;
      if (i < a.tiles) row[i] = pre;
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

// Stable scatter of one tile by one 8-bit digit.  Each wave ranks a contiguous quarter of the
// tile with ballots, the tile is reordered in LDS, then written out in digit runs.
template <bool FIRST>
__global__ __launch_bounds__(kBlock) void k_sort_scatter(SortArgs a) {
  __shared__ uint32_t s_key[kTile];
  __shared__ uint32_t s_val[kTile];
  __shared__ uint32_t s_wcnt[kWaves][256];
  __shared__ uint32_t s_gbase[256];
  __shared__ uint32_t s_lstart[256];
  __shared__ uint32_t s_w[kWaves];
  __shared__ int32_t s_off[FIRST ? kOffStage + 1 : 1];
  __shared__ int32_t s_jlo, s_jhi;

  const int tid = threadIdx.x, w = tid >> 6, lane = lane_id();
  const int t = blockIdx.x;
  const int32_t i0 = t * kTile;
  const int32_t tn = min(kTile, a.n - i0);

  // global start of each digit: digits below it over all tiles, plus this digit in earlier tiles
  {
    uint32_t total;
    const uint32_t below = block_excl_scan(a.tot[tid], s_w, total);
    s_gbase[tid] = below + a.counts[(size_t)tid * a.tiles + t];
    for (int ww = 0; ww < kWaves; ++ww) s_wcnt[ww][tid] = 0;
  }
  bool stage = false;
  if (FIRST) {
    if (tid == 0) {
      s_jlo = bag_search_global(a.offsets, 0, a.n_bags - 1, i0);
      s_jhi = bag_search_global(a.offsets, 0, a.n_bags - 1, i0 + tn - 1);
    }
    __syncthreads();
    stage = (s_jhi - s_jlo + 2) <= kOffStage + 1;
    if (stage)
      for (int i = tid; i <= s_jhi - s_jlo + 1; i += kBlock) s_off[i] = a.offsets[s_jlo + i];
  }
  __syncthreads();

  uint32_t key[kIPT], val[kIPT], rank[kIPT];
  const uint64_t lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int k = 0; k < kIPT; ++k) {
    const int32_t li = w * (kIPT * 64) + k * 64 + lane;  // item index inside the tile
    const bool valid = li < tn;
    const int32_t i = i0 + li;
    uint32_t kk = 0, vv = 0;
    if (valid) {
      if (FIRST) {
        kk = first_key(a.rowref[i], a.miss_key);
        if (stage) {
          int lo = 0, hi = s_jhi - s_jlo;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= i) lo = mid; else hi = mid - 1;
          }
          vv = (uint32_t)(s_jlo + lo);
        } else {
          vv = (uint32_t)bag_search_global(a.offsets, s_jlo, s_jhi, i);
        }
      } else {
        kk = a.kin[i];
        vv = a.vin[i];
      }
    }
    const uint32_t dg = (kk >> a.shift) & 255u;
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const uint64_t bb = __ballot((dg >> bit) & 1u);
      m &= ((dg >> bit) & 1u) ? bb : ~bb;
    }
    const uint32_t before = s_wcnt[w][dg];
    if (valid && (m & lt) == 0) s_wcnt[w][dg] = before + (uint32_t)__popcll(m);
    rank[k] = before + (uint32_t)__popcll(m & lt);
    key[k] = kk;
    val[k] = vv;
  }
  __syncthreads();
  // per digit: counts in earlier waves and the tile-local start
  {
    uint32_t c = 0;
    for (int ww = 0; ww < kWaves; ++ww) {
      const uint32_t x = s_wcnt[ww][tid];
      s_wcnt[ww][tid] = c;
      c += x;
    }
    uint32_t total;
    s_lstart[tid] = block_excl_scan(c, s_w, total);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kIPT; ++k) {
    const int32_t li = w * (kIPT * 64) + k * 64 + lane;
    if (li < tn) {
      const uint32_t dg = (key[k] >> a.shift) & 255u;
      const uint32_t p = s_lstart[dg] + s_wcnt[w][dg] + rank[k];
      s_key[p] = key[k];
      s_val[p] = val[k];
    }
  }
  __syncthreads();
  for (int p = tid; p < tn; p += kBlock) {
    const uint32_t kk = s_key[p];
    const uint32_t dg = (kk >> a.shift) & 255u;
    const uint32_t dst = s_gbase[dg] + ((uint32_t)p - s_lstart[dg]);
    a.kout[dst] = kk;
    a.vout[dst] = s_val[p];
  }
}

// ---------------------------------------------------------------- backward: reduce + Adagrad
struct UpdArgs {
  DevDesc d;
  const uint32_t* key;   // sorted rowrefs (miss_key last)
  const uint32_t* val;   // bag of each sorted occurrence
  int32_t n;
  uint32_t miss_key;
  const void* grad;
  float lr, eps;
  uint32_t* ctr;         // [0] long-segment count, [1] unique count
  uint32_t* long_list;
  int64_t* n_unique;
};

template <typename RowT, int EPL>
__device__ __forceinline__ void adagrad_row(const UpdArgs& a, uint32_t r, int e0,
                                            typename F32V<EPL>::t g) {
  typedef typename F32V<EPL>::t V;
  const uint64_t e = (uint64_t)r * a.d.granule + e0;
  V acc = load_f32<float, EPL>(a.d.acc + e);
  acc += g * g;
  V den;
#pragma unroll
  for (int q = 0; q < EPL; ++q) den[q] = __builtin_sqrtf(acc[q]) + a.eps;
  const V delta = (a.lr * g) / den;
  store_from_f32<float, EPL>(a.d.acc + e, acc);
  RowT* rows = reinterpret_cast<RowT*>(a.d.rows);
  if constexpr (sizeof(RowT) == 4) {
    V w = load_f32<RowT, EPL>(rows + e);
    store_from_f32<RowT, EPL>(rows + e, w - delta);
  } else if (a.d.has_master) {
    V m = load_f32<float, EPL>(a.d.master + e) - delta;
    store_from_f32<float, EPL>(a.d.master + e, m);
    store_from_f32<RowT, EPL>(rows + e, m);
  } else {
    V w = load_f32<RowT, EPL>(rows + e);
    store_from_f32<RowT, EPL>(rows + e, w - delta);
  }
}

// Each group of 2^gs_log2 lanes owns kQ consecutive sorted occurrences and every segment that
// starts among them.  Segments of at most kLong occurrences are reduced and updated here; longer
// ones are queued for k_update_long.
template <typename RowT, typename GradT>
__global__ __launch_bounds__(kBlock) void k_update_short(UpdArgs a, int gs_log2) {
  constexpr int EPL = 16 / (int)sizeof(RowT);
  typedef typename F32V<EPL>::t V;
  __shared__ uint32_t s_cnt;
  if (threadIdx.x == 0) s_cnt = 0;
  __syncthreads();
  const int lane = threadIdx.x & ((1 << gs_log2) - 1);
  const int64_t grp = ((int64_t)blockIdx.x * kBlock + threadIdx.x) >> gs_log2;
  const int64_t c0 = grp * kQ;
  const GradT* G = reinterpret_cast<const GradT*>(a.grad);
  const int F = a.d.n_fields;
  const int e0 = lane * EPL;
  uint32_t heads = 0;
  if (c0 < a.n) {
    const int32_t c1 = (int32_t)min<int64_t>(a.n, c0 + kQ);
    uint32_t prev = c0 > 0 ? a.key[c0 - 1] : 0xFFFFFFFFu;
    for (int32_t i = (int32_t)c0; i < c1; ++i) {
      const uint32_t k = a.key[i];
      if (k == a.miss_key) break;
      const bool head = (i == 0) || (k != prev);
      prev = k;
      if (!head) continue;
      ++heads;
      if (i + kLong < a.n && a.key[i + kLong] == k) {
        if (lane == 0) a.long_list[atomicAdd(&a.ctr[0], 1u)] = (uint32_t)i;
        continue;
      }
      const uint32_t bag0 = a.val[i];
      const int f = (int)(bag0 % (uint32_t)F);
      const int D = a.d.var_dim ? a.d.fdim[f] : a.d.fixed_dim;
      if (e0 >= D) continue;
      const int col = a.d.var_dim ? a.d.fcol[f] : f * a.d.fixed_dim;
      const GradT* Gc = G + col + e0;
      V g = 0.0f;
      int32_t e = i;
      for (;;) {
        uint32_t bg[4];
        bool ok[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          ok[u] = (e + u < a.n) && (a.key[e + u] == k);
          bg[u] = ok[u] ? a.val[e + u] : 0u;
        }
        V x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          x[u] = ok[u] ? load_f32<GradT, EPL>(Gc + (uint64_t)(bg[u] / (uint32_t)F) * a.d.out_width)
                       : V(0.0f);
#pragma unroll
        for (int u = 0; u < 4; ++u) g += x[u];
        if (!ok[3]) break;
        e += 4;
      }
      adagrad_row<RowT, EPL>(a, k, e0, g);
    }
  }
  if (lane == 0 && heads) atomicAdd(&s_cnt, heads);
  __syncthreads();
  if (threadIdx.x == 0 && s_cnt) atomicAdd(&a.ctr[1], s_cnt);
}

// One block per long segment: every lane group strides through the segment, partial sums meet in
// LDS, and one group applies the update.
template <typename RowT, typename GradT>
__global__ __launch_bounds__(kBlock) void k_update_long(UpdArgs a, int gs_log2) {
  constexpr int EPL = 16 / (int)sizeof(RowT);
  typedef typename F32V<EPL>::t V;
  __shared__ V s_part[kBlock];
  const int lane = threadIdx.x & ((1 << gs_log2) - 1);
  const int grp = threadIdx.x >> gs_log2;
  const int ngrp = kBlock >> gs_log2;
  const GradT* G = reinterpret_cast<const GradT*>(a.grad);
  const int F = a.d.n_fields;
  const int e0 = lane * EPL;
  const uint32_t n_long = a.ctr[0];
  if (blockIdx.x == 0 && threadIdx.x == 0 && a.n_unique) *a.n_unique = (int64_t)a.ctr[1];
  for (uint32_t s = blockIdx.x; s < n_long; s += gridDim.x) {
    const int32_t i0 = (int32_t)a.long_list[s];
    const uint32_t k = a.key[i0];
    const uint32_t bag0 = a.val[i0];
    const int f = (int)(bag0 % (uint32_t)F);
    const int D = a.d.var_dim ? a.d.fdim[f] : a.d.fixed_dim;
    const int col = a.d.var_dim ? a.d.fcol[f] : f * a.d.fixed_dim;
    const GradT* Gc = G + col + e0;
    V g = 0.0f;
    if (e0 < D) {
      int32_t e = i0 + grp;
      for (;;) {
        uint32_t bg[4];
        bool ok[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int32_t x = e + u * ngrp;
          ok[u] = (x < a.n) && (a.key[x] == k);
          bg[u] = ok[u] ? a.val[x] : 0u;
        }
        V x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          x[u] = ok[u] ? load_f32<GradT, EPL>(Gc + (uint64_t)(bg[u] / (uint32_t)F) * a.d.out_width)
                       : V(0.0f);
#pragma unroll
        for (int u = 0; u < 4; ++u) g += x[u];
        if (!ok[3]) break;
        e += 4 * ngrp;
      }
    }
    s_part[threadIdx.x] = g;
    __syncthreads();
    if (grp == 0 && e0 < D) {
      V tot = 0.0f;
      for (int q = 0; q < ngrp; ++q) tot += s_part[(q << gs_log2) + lane];
      adagrad_row<RowT, EPL>(a, k, e0, tot);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- optional unique list output
struct SegArgs {
  const uint32_t* key;
  int32_t n;
  int32_t tiles;
  uint32_t miss_key;
  uint32_t* seg;      // [tiles + 1] head counts -> exclusive offsets; [tiles] = U
  uint32_t* headpos;  // [n + 1] position of each head
  uint32_t* unique;
  int32_t* count;
  uint32_t* nvalid;   // one word: number of non-miss occurrences
};

__device__ __forceinline__ bool seg_head(const SegArgs& a, int32_t i) {
  const uint32_t k = a.key[i];
  return k != a.miss_key && (i == 0 || a.key[i - 1] != k);
}

__global__ __launch_bounds__(kBlock) void k_seg_count(SegArgs a) {
  __shared__ uint32_t s_c, s_v;
  if (threadIdx.x == 0) { s_c = 0; s_v = 0; }
  __syncthreads();
  const int32_t i0 = blockIdx.x * kTile, i1 = min(a.n, i0 + kTile);
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
  const int32_t i0 = blockIdx.x * kTile;
  uint32_t base = a.seg[blockIdx.x];
  for (int32_t c = 0; c < kTile; c += kBlock) {
    const int32_t i = i0 + c + threadIdx.x;
    const bool h = (i < a.n) && seg_head(a, i);
    uint32_t total;
    const uint32_t pre = block_excl_scan(h ? 1u : 0u, s_w, total);
    if (h) {
      a.unique[base + pre] = a.key[i];
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
  (void)hipEventRecord(r->a, c.stream);
}
KTimer::~KTimer() {
  if (r) (void)hipEventRecord(r->b, c.stream);
}

hipError_t launch_lookup_pool(const FwdLaunch& a, LaunchCtx& ctx) {
  if (a.n_bags <= 0) return hipSuccess;
  const int gs = log2_group(a.d.max_dim, a.d.row_f16 ? 8 : 4);
  const dim3 grid((a.n_bags + kFwdBags - 1) / kFwdBags);
  KTimer tm(ctx, "lookup_pool");
  if (a.d.row_f16) {
    if (a.out_f16)
      hipLaunchKernelGGL((k_lookup_pool<_Float16, _Float16>), grid, dim3(kBlock), 0, ctx.stream, a, gs);
    else
      hipLaunchKernelGGL((k_lookup_pool<_Float16, float>), grid, dim3(kBlock), 0, ctx.stream, a, gs);
  } else {
    if (a.out_f16)
      hipLaunchKernelGGL((k_lookup_pool<float, _Float16>), grid, dim3(kBlock), 0, ctx.stream, a, gs);
    else
      hipLaunchKernelGGL((k_lookup_pool<float, float>), grid, dim3(kBlock), 0, ctx.stream, a, gs);
  }
  return hipGetLastError();
}

BwdPlan plan_bwd(int64_t nnz, uint32_t rowref_space) {
  BwdPlan p{};
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.n = (int32_t)nnz;
  p.tiles = (int32_t)((nnz + kTile - 1) / kTile);
  p.miss_key = rowref_space;
  int bits = 0;
  while (bits < 32 && (uint64_t)(p.miss_key >> bits) != 0) ++bits;
  p.passes = bits <= 8 ? 1 : (bits + 7) / 8;
  const size_t n = (size_t)(nnz > 0 ? nnz : 0);
  size_t o = 0;
  p.off_ka = o; o = al(o + 4 * (n + 1));
  p.off_va = o; o = al(o + 4 * (n + 1));
  p.off_kb = o; o = al(o + 4 * (n + 1));
  p.off_vb = o; o = al(o + 4 * (n + 1));
  p.off_counts = o; o = al(o + 4 * (size_t)256 * (size_t)(p.tiles > 0 ? p.tiles : 1));
  p.off_tot = o; o = al(o + 4 * 256);
  p.off_ctr = o; o = al(o + 4 * 16);
  p.off_long = o; o = al(o + 4 * (n / (kLong + 1) + 1));
  p.off_seg = o; o = al(o + 4 * ((size_t)p.tiles + 1));
  p.bytes = o;
  return p;
}

hipError_t launch_adagrad_bwd(const BwdLaunch& a, const BwdPlan& p, LaunchCtx& ctx) {
  uint8_t* ws = reinterpret_cast<uint8_t*>(a.ws);
  uint32_t* ctr = reinterpret_cast<uint32_t*>(ws + p.off_ctr);
  if (p.n <= 0) {
    if (a.n_unique) {
      KTimer tm(ctx, "set_n_unique");
      hipLaunchKernelGGL(k_set_i64, dim3(1), dim3(1), 0, ctx.stream, a.n_unique, (int64_t)0);
    }
    return hipGetLastError();
  }
  SortArgs s{};
  s.rowref = a.rowref;
  s.offsets = a.offsets;
  s.n_bags = a.n_bags;
  s.counts = reinterpret_cast<uint32_t*>(ws + p.off_counts);
  s.tot = reinterpret_cast<uint32_t*>(ws + p.off_tot);
  s.ctr = ctr;
  s.n = p.n;
  s.tiles = p.tiles;
  s.miss_key = p.miss_key;
  uint32_t* ka = reinterpret_cast<uint32_t*>(ws + p.off_ka);
  uint32_t* va = reinterpret_cast<uint32_t*>(ws + p.off_va);
  uint32_t* kb = reinterpret_cast<uint32_t*>(ws + p.off_kb);
  uint32_t* vb = reinterpret_cast<uint32_t*>(ws + p.off_vb);
  const dim3 tiles(p.tiles), blk(kBlock);
  uint32_t *src_k = nullptr, *src_v = nullptr, *dst_k = ka, *dst_v = va;
  for (int pass = 0; pass < p.passes; ++pass) {
    s.shift = 8 * pass;
    s.kin = src_k;
    s.vin = src_v;
    s.kout = dst_k;
    s.vout = dst_v;
    {
      KTimer tm(ctx, "sort_hist");
      if (pass == 0) hipLaunchKernelGGL(k_sort_hist<true>, tiles, blk, 0, ctx.stream, s);
      else hipLaunchKernelGGL(k_sort_hist<false>, tiles, blk, 0, ctx.stream, s);
    }
    {
      KTimer tm(ctx, "sort_scan");
      hipLaunchKernelGGL(k_sort_scan, dim3(256), blk, 0, ctx.stream, s, pass == 0 ? 1 : 0);
    }
    {
      KTimer tm(ctx, "sort_scatter");
      if (pass == 0) hipLaunchKernelGGL(k_sort_scatter<true>, tiles, blk, 0, ctx.stream, s);
      else hipLaunchKernelGGL(k_sort_scatter<false>, tiles, blk, 0, ctx.stream, s);
    }
    src_k = dst_k;
    src_v = dst_v;
    dst_k = (src_k == ka) ? kb : ka;
    dst_v = (src_v == va) ? vb : va;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  UpdArgs u{};
  u.d = a.d;
  u.key = src_k;
  u.val = src_v;
  u.n = p.n;
  u.miss_key = p.miss_key;
  u.grad = a.grad;
  u.lr = a.lr;
  u.eps = a.eps;
  u.ctr = ctr;
  u.long_list = reinterpret_cast<uint32_t*>(ws + p.off_long);
  u.n_unique = a.n_unique;
  const int epl = a.d.row_f16 ? 8 : 4;
  const int gsl = log2_group(a.d.max_dim, epl);
  const int64_t groups = ((int64_t)p.n + kQ - 1) / kQ;
  const int64_t per_block = kBlock >> gsl;
  const dim3 gshort((unsigned)((groups + per_block - 1) / per_block));
  const int64_t max_long = (int64_t)p.n / (kLong + 1) + 1;
  const dim3 glong((unsigned)(max_long < 4096 ? max_long : 4096));
  {
    KTimer tm(ctx, "update_short");
    if (a.d.row_f16) {
      if (a.grad_f16) hipLaunchKernelGGL((k_update_short<_Float16, _Float16>), gshort, blk, 0, ctx.stream, u, gsl);
      else hipLaunchKernelGGL((k_update_short<_Float16, float>), gshort, blk, 0, ctx.stream, u, gsl);
    } else {
      if (a.grad_f16) hipLaunchKernelGGL((k_update_short<float, _Float16>), gshort, blk, 0, ctx.stream, u, gsl);
      else hipLaunchKernelGGL((k_update_short<float, float>), gshort, blk, 0, ctx.stream, u, gsl);
    }
  }
  {
    KTimer tm(ctx, "update_long");
    if (a.d.row_f16) {
      if (a.grad_f16) hipLaunchKernelGGL((k_update_long<_Float16, _Float16>), glong, blk, 0, ctx.stream, u, gsl);
      else hipLaunchKernelGGL((k_update_long<_Float16, float>), glong, blk, 0, ctx.stream, u, gsl);
    } else {
      if (a.grad_f16) hipLaunchKernelGGL((k_update_long<float, _Float16>), glong, blk, 0, ctx.stream, u, gsl);
      else hipLaunchKernelGGL((k_update_long<float, float>), glong, blk, 0, ctx.stream, u, gsl);
    }
  }
  err = hipGetLastError();
  if (err != hipSuccess || !a.unique) return err;

  SegArgs g{};
  g.key = src_k;
  g.n = p.n;
  g.tiles = p.tiles;
  g.miss_key = p.miss_key;
  g.seg = reinterpret_cast<uint32_t*>(ws + p.off_seg);
  g.headpos = dst_k;  // the spare key buffer (n + 1 words)
  g.unique = a.unique;
  g.count = a.count;
  g.nvalid = ctr + 2;
  {
    KTimer tm(ctx, "seg_zero");
    hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(64), 0, ctx.stream, ctr + 2, 1);
  }
  {
    KTimer tm(ctx, "seg_count");
    hipLaunchKernelGGL(k_seg_count, tiles, blk, 0, ctx.stream, g);
  }
  {
    KTimer tm(ctx, "seg_scan");
    hipLaunchKernelGGL(k_seg_scan, dim3(1), blk, 0, ctx.stream, g);
  }
  {
    KTimer tm(ctx, "seg_write");
    hipLaunchKernelGGL(k_seg_write, tiles, blk, 0, ctx.stream, g);
  }
  if (a.count) {
    KTimer tm(ctx, "seg_counts");
    hipLaunchKernelGGL(k_seg_counts, dim3(1024), blk, 0, ctx.stream, g);
  }
  return hipGetLastError();
}

}  // namespace emb
