// Top-k selection over the visible index scores (Evidence Ledger Eqs 13-17:
// the top-k scores pick the compressed blocks the core attention reads).
//
// One block per query row.  Scores map to order-preserving unsigned keys.  An
// MSB-first radix select with LDS histograms finds the k-th largest key K*;
// then every entry with key > K* and the lowest-index entries with key == K*
// (until k are taken) are written in ascending entry order, so ties go to the
// lower index, and rows with fewer than k visible entries are padded with -1.
//
// Rows of up to 16 * 1024 entries run in one block per row with the keys in
// registers: thread t owns the contiguous entries [16 t, 16 t + 16).  The
// first digit is counted block-wide; the keys sharing it with the k-th largest
// (the candidates) are compacted into LDS and one wave resolves the remaining
// digits over them alone (past TK_CAND_CAP candidates the block resolves them
// over the keys in registers instead); the ordered compaction is a single
// block-wide scan.  Longer rows spread over many blocks per row: bf16 scores
// (decode rows of up to 2^24 entries) in two launches -- per-slice 16-bit key
// histograms kept above each slice's own k-th largest key, then per slice the
// row's K* and the slice's ordered write -- and fp32 scores by a per-digit
// sequence of slice histograms and per-row reductions, then per-slice counts
// and an ordered emit at each slice's offset.
#include "common.hpp"
#include "internal.hpp"

namespace csa {

// larger score -> larger key; NaN never occurs
__device__ __forceinline__ uint32_t f32_key(uint32_t u) {
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint32_t bf16_key(uint32_t u) {
  return (u & 0x8000u) ? (~u & 0xFFFFu) : (u | 0x8000u);
}

template <bool BF16>
__device__ __forceinline__ uint32_t load_key(const void* scores, int64_t i) {
  if (BF16) return bf16_key(reinterpret_cast<const uint16_t*>(scores)[i]);
  return f32_key(reinterpret_cast<const uint32_t*>(scores)[i]);
}

// the 16 keys of entries [s0, s0 + 16) of a row (0 for s >= nv); whole
// 16-byte loads when the chunk lies inside the row's Nmax entries
template <bool BF16>
__device__ __forceinline__ void load_keys16(const void* srow, int s0, int nv, int Nmax,
                                            uint32_t* key) {
  if (s0 + 16 <= Nmax) {
    if (BF16) {
      const u32x4* p = reinterpret_cast<const u32x4*>((const uint16_t*)srow + s0);
      const u32x4 a = p[0], b = p[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        key[2 * i] = bf16_key(a[i] & 0xFFFFu);
        key[2 * i + 1] = bf16_key(a[i] >> 16);
        key[8 + 2 * i] = bf16_key(b[i] & 0xFFFFu);
        key[8 + 2 * i + 1] = bf16_key(b[i] >> 16);
      }
    } else {
      const u32x4* p = reinterpret_cast<const u32x4*>((const uint32_t*)srow + s0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 v = p[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) key[4 * j + i] = f32_key(v[i]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) key[i] = (s0 + i < Nmax) ? load_key<BF16>(srow, s0 + i) : 0u;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (s0 + i >= nv) key[i] = 0u;
}

// Wave-wide helpers on DPP row moves (no LDS round trips); every lane of the
// wave must be active.  DPP controls: quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] =
// 0x4E, row_ror:n = 0x120 + n, row_shr:n = 0x110 + n.
template <int CTRL>
__device__ __forceinline__ int dpp_move(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ int wave_all_max(int x) {
  x = max(x, dpp_move<0xB1>(x));
  x = max(x, dpp_move<0x4E>(x));
  x = max(x, dpp_move<0x124>(x));
  x = max(x, dpp_move<0x128>(x));  // every lane holds its row's maximum
  const int a = max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16));
  const int b = max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48));
  return max(a, b);
}
__device__ __forceinline__ int wave_all_min(int x) { return -wave_all_max(-x); }
// inclusive prefix sum over the lanes of the wave
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += dpp_move<0x111>(x);
  x += dpp_move<0x112>(x);
  x += dpp_move<0x114>(x);
  x += dpp_move<0x118>(x);  // prefix within each row of 16 lanes
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  const int lane = threadIdx.x & 63;
  return x + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
}

// exclusive block scan of one int per thread; *total gets the block sum.  `ws`
// is LDS of >= 16 ints, not written again before a later barrier (one barrier
// here).  Every thread of the block must call.
__device__ __forceinline__ int block_scan_excl(int v, int* ws, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int incl = wave_incl_sum(v);
  if (lane == 63) ws[wave] = incl;
  __syncthreads();
  int pre = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const int y = ws[i];
    pre += (i < wave) ? y : 0;
    tot += y;
  }
  *total = tot;
  return incl - v + pre;
}

// Locate the digit of the `remaining`-th largest key among the keys counted in
// hist[0..nbins) (descending digits).  Wave 0 scans; the digit and the count of
// keys in larger digits land in *digit / *above.  nbins is a multiple of 64.
__device__ __forceinline__ void find_digit(const int* hist, int nbins, int remaining,
                                           uint32_t* digit, int* above) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const int per = nbins / 64;
  const int top = nbins - 1 - per * lane;  // this lane scans digits top .. top-per+1
  int cnt = 0;
  for (int i = 0; i < per; ++i) cnt += hist[top - i];
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  const int excl = incl - cnt;
  if (excl < remaining && incl >= remaining) {
    int acc = excl;
    for (int i = 0; i < per; ++i) {
      const int h = hist[top - i];
      if (acc + h >= remaining) {
        *digit = (uint32_t)(top - i);
        *above = acc;
        break;
      }
      acc += h;
    }
  }
}

// Block-wide version of find_digit for large histograms: thread t owns the
// nbins / blockDim digits just below those of thread t-1 (descending), one
// block scan orders the ranges, and the thread whose range holds the rank
// scans it.  Every thread of the block must call.
__device__ __forceinline__ void find_digit_block(const int* hist, int nbins, int remaining,
                                                 int* scan_ws, uint32_t* digit, int* above) {
  const int per = nbins / blockDim.x;
  const int top = nbins - 1 - per * threadIdx.x;
  int cnt = 0;
  for (int i = 0; i < per; ++i) cnt += hist[top - i];
  int total;
  const int excl = block_scan_excl(cnt, scan_ws, &total);
  if (excl < remaining && excl + cnt >= remaining) {
    int acc = excl;
    for (int i = 0; i < per; ++i) {
      const int h = hist[top - i];
      if (acc + h >= remaining) {
        *digit = (uint32_t)(top - i);
        *above = acc;
        break;
      }
      acc += h;
    }
  }
}

// exclusive prefix of one int per lane within the wave; *total gets the wave
// sum.  Every lane of the wave must call.
__device__ __forceinline__ int wave_scan_excl(int v, int* total) {
  const int incl = wave_incl_sum(v);
  *total = __builtin_amdgcn_readlane(incl, 63);
  return incl - v;
}

// candidates compacted for the last digits (more go the block-wide way): a
// small buffer keeps more rows resident per CU when many short rows run
constexpr int TK_CAND_CAP = 2048;

// W1: width of the first digit of fp32 keys (13, or 12 when many rows share the
// GPU: a 16 KB histogram lets four 512-thread blocks reside per CU instead of
// three).  bf16 keys take 10 then 6 bits.
template <bool BF16, int W1>
__device__ __forceinline__ void topk_row(const void* __restrict__ scores,
                                         const int32_t* __restrict__ q_pos,
                                         const int32_t* __restrict__ n_entries, int Tq, int Nmax,
                                         int m, int k, int vec, int32_t* __restrict__ idx) {
  __shared__ int hist[BF16 ? 1024 : (1 << W1)];
  extern __shared__ uint32_t cand[];  // [min(16 * blockDim, TK_CAND_CAP)]: keys sharing the k-th's first digit
  __shared__ int scan_ws[16];
  __shared__ uint32_t sh_digit;
  __shared__ int sh_above, sh_ncand;
  const int row = blockIdx.x, b = row / Tq;
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63;
  const int cap = min(16 * nt, TK_CAND_CAP);
  int32_t* out = idx + (int64_t)row * k;
  const void* srow = BF16 ? (const void*)((const uint16_t*)scores + (int64_t)row * Nmax)
                          : (const void*)((const uint32_t*)scores + (int64_t)row * Nmax);
  // ---- keys in registers: thread t owns entries [16 t, 16 t + 16).  Whole
  // 16-byte loads leave before the row's visible count is known (their latency
  // overlaps its loads); the keys are formed and masked after it
  const int s0 = tid * 16;
  const bool whole = vec && s0 + 16 <= Nmax;
  u32x4 raw[BF16 ? 2 : 4];
  if (whole) {
    const u32x4* p = reinterpret_cast<const u32x4*>(
        BF16 ? (const void*)((const uint16_t*)srow + s0) : (const void*)((const uint32_t*)srow + s0));
#pragma unroll
    for (int j = 0; j < (BF16 ? 2 : 4); ++j) raw[j] = p[j];
  }
  const int nv = min(min(n_entries[b], Nmax), (q_pos[row] + 1) / m);
  if (nv <= k) {
    for (int i = tid; i < k; i += nt) out[i] = i < nv ? i : -1;
    return;
  }
  uint32_t key[16];
  if (whole) {
#pragma unroll
    for (int j = 0; j < (BF16 ? 2 : 4); ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (BF16) {
          key[8 * j + 2 * i] = bf16_key(raw[j][i] & 0xFFFFu);
          key[8 * j + 2 * i + 1] = bf16_key(raw[j][i] >> 16);
        } else {
          key[4 * j + i] = f32_key(raw[j][i]);
        }
      }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (s0 + i >= nv) key[i] = 0u;
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) key[i] = (s0 + i < nv) ? load_key<BF16>(srow, s0 + i) : 0u;
  }
  // ---- first digit, block-wide: W1 bits of fp32 keys (bits 31..32-W1), 10 of
  // bf16 (15..6); wide digits spread the clustered score exponents over many bins
  constexpr int SH1 = BF16 ? 6 : 32 - W1;
  constexpr int NB1 = 1 << (BF16 ? 10 : W1);
  for (int i = tid; i < NB1; i += nt) hist[i] = 0;
  if (tid == 0) sh_ncand = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (s0 + i < nv) atomicAdd(&hist[key[i] >> SH1], 1);
  __syncthreads();
  find_digit_block(hist, NB1, k, scan_ws, &sh_digit, &sh_above);
  __syncthreads();
  const uint32_t d1 = sh_digit;
  int remaining = k - sh_above;  // rank to locate among the keys of digit d1
  // ---- candidates: keys of digit d1, appended to LDS (one atomic per wave)
  {
    int mine = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) mine += (s0 + i < nv && (key[i] >> SH1) == d1) ? 1 : 0;
    int wtot;
    int pos = wave_scan_excl(mine, &wtot);
    int base = 0;
    if (lane == 0 && wtot) base = atomicAdd(&sh_ncand, wtot);
    pos += __shfl(base, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (s0 + i < nv && (key[i] >> SH1) == d1) {
        if (pos < cap) cand[pos] = key[i];
        ++pos;
      }
  }
  __syncthreads();
  const int nc = sh_ncand;
  if (nc > cap) {
    // ---- too many candidates to compact: the remaining digits block-wide over
    // the keys in registers (same digits, same rule)
    uint32_t prefix = d1 << SH1, pmask = ~0u << SH1;
    int shift = SH1;
    while (shift > 0) {
      const int width = BF16 ? 6 : min(shift, 10);
      shift -= width;
      const int nbins = 1 << width;
      const uint32_t dmask = (uint32_t)nbins - 1u;
      for (int i = tid; i < nbins; i += nt) hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (s0 + i < nv && (key[i] & pmask) == prefix) atomicAdd(&hist[(key[i] >> shift) & dmask], 1);
      __syncthreads();
      find_digit(hist, nbins, remaining, &sh_digit, &sh_above);
      __syncthreads();
      const uint32_t dg = sh_digit;
      remaining -= sh_above;
      prefix |= dg << shift;
      pmask |= dmask << shift;
      __syncthreads();  // every thread has read this digit
    }
    if (tid == 0) {
      sh_digit = prefix;
      sh_above = remaining;
    }
  } else if (tid < 64) {
    // ---- remaining digits over the candidates by wave 0 alone (no block
    // barriers), at most 6 bits each: one bin per lane, located by a prefix
    // sum over the lanes (fp32 keys 20 or 19 bits in 4 digits, bf16 keys 6)
    uint32_t prefix = d1 << SH1, pmask = ~0u << SH1;
    int shift = SH1;
    while (shift > 0) {
      const int width = min(shift, 6);
      shift -= width;
      const int nbins = 1 << width;
      const uint32_t dmask = (uint32_t)nbins - 1u;
      hist[lane] = 0;
      __builtin_amdgcn_wave_barrier();
      for (int i = lane; i < nc; i += 64) {
        const uint32_t kk = cand[i];
        if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & dmask], 1);
      }
      __builtin_amdgcn_wave_barrier();
      // lane j takes digit nbins - 1 - j: descending digits
      const int c = lane < nbins ? hist[nbins - 1 - lane] : 0;
      const int incl = wave_incl_sum(c);
      const uint64_t hit = __ballot(incl - c < remaining && incl >= remaining);
      const int j = (int)__builtin_ctzll(hit) & 63;
      remaining -= __builtin_amdgcn_readlane(incl - c, j);
      prefix |= (uint32_t)(nbins - 1 - j) << shift;
      pmask |= dmask << shift;
      __builtin_amdgcn_wave_barrier();  // the bins are read before the next digit clears them
    }
    if (lane == 0) {
      sh_digit = prefix;
      sh_above = remaining;
    }
  }
  __syncthreads();
  const uint32_t kstar = sh_digit;
  const int need_eq = sh_above;  // entries equal to K* to take, lowest index first
  // ---- ordered compaction: one block-wide scan of (above, equal) counts
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bool ok = s0 + i < nv;
    gt += (ok && key[i] > kstar) ? 1 : 0;
    eq += (ok && key[i] == kstar) ? 1 : 0;
  }
  int total;
  const int excl = block_scan_excl(gt | (eq << 16), scan_ws, &total);
  int gt_before = excl & 0xFFFF, eq_before = excl >> 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bool ok = s0 + i < nv;
    const bool g = ok && key[i] > kstar, e = ok && key[i] == kstar;
    if (g || (e && eq_before < need_eq)) {
      const int pos = gt_before + min(eq_before, need_eq);
      if (pos < k) out[pos] = s0 + i;
    }
    gt_before += g ? 1 : 0;
    eq_before += e ? 1 : 0;
  }
}

template <bool BF16, int W1>
__global__ __launch_bounds__(1024) void topk_kernel(const void* __restrict__ scores,
                                                    const int32_t* __restrict__ q_pos,
                                                    const int32_t* __restrict__ n_entries, int Tq,
                                                    int Nmax, int m, int k, int vec,
                                                    int32_t* __restrict__ idx) {
  topk_row<BF16, W1>(scores, q_pos, n_entries, Tq, Nmax, m, k, vec, idx);
}

// many rows of fp32 scores (prefill): held to 64 registers so that four
// 512-thread blocks reside per CU (measured: 32K prefill 389 -> 350 us; the
// few-row kernel above stays unconstrained, which is faster for decode)
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(8))) void topk_many_kernel(
    const void* __restrict__ scores, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int Nmax, int m, int k, int vec,
    int32_t* __restrict__ idx) {
  topk_row<false, 12>(scores, q_pos, n_entries, Tq, Nmax, m, k, vec, idx);
}

// ------------------------------------------------------------------ long rows
// Multi-block radix select.  Row r is cut into P slices of TKM_SLICE entries,
// one 256-thread block each (16 keys per thread in registers).  Per digit:
// topk_hist_kernel writes each slice's histogram of the digit among the keys
// that match the row's current prefix; topk_reduce_kernel sums them, locates
// the digit holding the remaining rank and extends the prefix.  After the last
// digit the prefix is the k-th largest key K* and `remaining` the number of
// keys equal to K* to take; topk_count_kernel counts each slice's keys above /
// equal to K* and topk_emit_kernel writes the slice's selection at its offset.
// Workspace (ints): row state [rows][4], histograms [rows][P][2048], counts
// [rows][P][2].
constexpr int TKM_THREADS = 256;
constexpr int TKM_SLICE = 16 * TKM_THREADS;

struct TkRow {
  uint32_t prefix, pmask;
  int remaining;
  int pad;
};

__device__ __forceinline__ int row_visible(const int32_t* q_pos, const int32_t* n_entries, int row,
                                           int Tq, int Nmax, int m) {
  return min(min(n_entries[row / Tq], Nmax), (q_pos[row] + 1) / m);
}

template <bool BF16>
__global__ __launch_bounds__(TKM_THREADS) void topk_hist_kernel(
    const void* __restrict__ scores, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int Nmax, int m, int k, int vec, int P,
    int shift, int width, const TkRow* __restrict__ st, int* __restrict__ hist) {
  __shared__ int h[2048];
  const int row = blockIdx.x / P, p = blockIdx.x % P, tid = threadIdx.x;
  const int nv = row_visible(q_pos, n_entries, row, Tq, Nmax, m);
  if (nv <= k) return;
  const int nbins = 1 << width;
  const uint32_t dmask = (uint32_t)nbins - 1u;
  const uint32_t prefix = st ? st[row].prefix : 0u, pmask = st ? st[row].pmask : 0u;
  for (int i = tid; i < nbins; i += TKM_THREADS) h[i] = 0;
  __syncthreads();
  const int s0 = p * TKM_SLICE + 16 * tid;
  if (s0 < nv) {
    const void* srow = BF16 ? (const void*)((const uint16_t*)scores + (int64_t)row * Nmax)
                            : (const void*)((const uint32_t*)scores + (int64_t)row * Nmax);
    uint32_t key[16];
    if (vec) {
      load_keys16<BF16>(srow, s0, nv, Nmax, key);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) key[i] = (s0 + i < nv) ? load_key<BF16>(srow, s0 + i) : 0u;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (s0 + i < nv && (key[i] & pmask) == prefix) atomicAdd(&h[(key[i] >> shift) & dmask], 1);
  }
  __syncthreads();
  int* out = hist + ((int64_t)row * P + p) * 2048;
  for (int i = tid; i < nbins; i += TKM_THREADS) out[i] = h[i];
}

// one block per row: sum the slice histograms, fix the digit
__global__ __launch_bounds__(1024) void topk_reduce_kernel(
    const int32_t* __restrict__ q_pos, const int32_t* __restrict__ n_entries, int Tq, int Nmax,
    int m, int k, int P, int shift, int width, int first, TkRow* __restrict__ st,
    const int* __restrict__ hist) {
  __shared__ int h[2048];
  __shared__ uint32_t sh_digit;
  __shared__ int sh_above;
  const int row = blockIdx.x, tid = threadIdx.x;
  const int nv = row_visible(q_pos, n_entries, row, Tq, Nmax, m);
  if (nv <= k) return;
  const int nbins = 1 << width;
  const int* hr = hist + (int64_t)row * P * 2048;
  // thread (bin, part): sums slices part, part + parts, ...; parts combine in LDS
  const int parts = nbins >= 1024 ? 1 : 1024 / nbins;
  for (int i = tid; i < nbins; i += 1024) h[i] = 0;
  __syncthreads();
  for (int i = tid; i < nbins * parts; i += 1024) {
    const int bin = i % nbins, part = i / nbins;
    int acc = 0;
#pragma unroll 8
    for (int p = part; p < P; p += parts) acc += hr[(int64_t)p * 2048 + bin];
    if (acc) atomicAdd(&h[bin], acc);
  }
  const TkRow cur = first ? TkRow{0u, 0u, k, 0} : st[row];
  __syncthreads();
  find_digit(h, nbins, cur.remaining, &sh_digit, &sh_above);
  __syncthreads();
  if (tid == 0) {
    TkRow nx;
    nx.prefix = cur.prefix | (sh_digit << shift);
    nx.pmask = cur.pmask | ((uint32_t)(nbins - 1) << shift);
    nx.remaining = cur.remaining - sh_above;
    nx.pad = 0;
    st[row] = nx;
  }
}

// per slice: keys above K* and keys equal to K*
template <bool BF16>
__global__ __launch_bounds__(TKM_THREADS) void topk_count_kernel(
    const void* __restrict__ scores, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int Nmax, int m, int k, int vec, int P,
    const TkRow* __restrict__ st, int* __restrict__ cnt) {
  __shared__ int scan_ws[16];
  const int row = blockIdx.x / P, p = blockIdx.x % P, tid = threadIdx.x;
  const int nv = row_visible(q_pos, n_entries, row, Tq, Nmax, m);
  if (nv <= k) return;
  const uint32_t kstar = st[row].prefix;
  const int s0 = p * TKM_SLICE + 16 * tid;
  int gt = 0, eq = 0;
  if (s0 < nv) {
    const void* srow = BF16 ? (const void*)((const uint16_t*)scores + (int64_t)row * Nmax)
                            : (const void*)((const uint32_t*)scores + (int64_t)row * Nmax);
    uint32_t key[16];
    if (vec) {
      load_keys16<BF16>(srow, s0, nv, Nmax, key);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) key[i] = (s0 + i < nv) ? load_key<BF16>(srow, s0 + i) : 0u;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      gt += (s0 + i < nv && key[i] > kstar) ? 1 : 0;
      eq += (s0 + i < nv && key[i] == kstar) ? 1 : 0;
    }
  }
  int total;
  block_scan_excl(gt | (eq << 16), scan_ws, &total);
  if (tid == 0) {
    int* c = cnt + ((int64_t)row * P + p) * 2;
    c[0] = total & 0xFFFF;
    c[1] = total >> 16;
  }
}

// per slice: ordered write of the slice's selection at its offset; rows with
// N(q) <= k take all their visible entries
template <bool BF16>
__global__ __launch_bounds__(TKM_THREADS) void topk_emit_kernel(
    const void* __restrict__ scores, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int Nmax, int m, int k, int vec, int P,
    const TkRow* __restrict__ st, const int* __restrict__ cnt, int32_t* __restrict__ idx) {
  __shared__ int scan_ws[16];
  __shared__ int sh_gt, sh_eq;
  const int row = blockIdx.x / P, p = blockIdx.x % P, tid = threadIdx.x;
  const int nv = row_visible(q_pos, n_entries, row, Tq, Nmax, m);
  int32_t* out = idx + (int64_t)row * k;
  if (nv <= k) {
    for (int i = p * TKM_THREADS + tid; i < k; i += P * TKM_THREADS) out[i] = i < nv ? i : -1;
    return;
  }
  const uint32_t kstar = st[row].prefix;
  const int need_eq = st[row].remaining;
  // offsets: selections of the slices before this one
  if (tid < 64) {
    int g = 0, e = 0;
    for (int q = tid; q < p; q += 64) {
      g += cnt[((int64_t)row * P + q) * 2];
      e += cnt[((int64_t)row * P + q) * 2 + 1];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      g += __shfl_xor(g, o);
      e += __shfl_xor(e, o);
    }
    if (tid == 0) {
      sh_gt = g;
      sh_eq = e;
    }
  }
  __syncthreads();
  const int s0 = p * TKM_SLICE + 16 * tid;
  uint32_t key[16];
  const void* srow = BF16 ? (const void*)((const uint16_t*)scores + (int64_t)row * Nmax)
                          : (const void*)((const uint32_t*)scores + (int64_t)row * Nmax);
  if (s0 < nv) {
    if (vec) {
      load_keys16<BF16>(srow, s0, nv, Nmax, key);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) key[i] = (s0 + i < nv) ? load_key<BF16>(srow, s0 + i) : 0u;
    }
  }
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bool ok = s0 + i < nv;
    gt += (ok && key[i] > kstar) ? 1 : 0;
    eq += (ok && key[i] == kstar) ? 1 : 0;
  }
  int total;
  const int excl = block_scan_excl(gt | (eq << 16), scan_ws, &total);
  int gt_before = sh_gt + (excl & 0xFFFF), eq_before = sh_eq + (excl >> 16);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bool ok = s0 + i < nv;
    const bool g = ok && key[i] > kstar, e = ok && key[i] == kstar;
    if (g || (e && eq_before < need_eq)) {
      const int pos = gt_before + min(eq_before, need_eq);
      if (pos < k) out[pos] = s0 + i;
    }
    gt_before += g ? 1 : 0;
    eq_before += e ? 1 : 0;
  }
}

// ------------------------------------------------------------------ long bf16 rows
// Rows of more than 16 * 1024 bf16 scores (decode at 1M context: 2^18 entries
// per row) in two launches over (row, slice) blocks; no block reads more than
// its own slice of TKF_SLICE entries.
//  1. topk_fine_hist_kernel counts the slice's 16-bit keys in an LDS histogram
//     (two 16-bit counters per word), finds the slice's own k-th largest key lo
//     (its smallest key when it holds fewer than k) and its largest key hi, and
//     stores lo, hi, its entry count and the histogram over [lo, hi].  A slice
//     with k or more entries holds k keys >= its lo, so the row's k-th largest
//     key K* is at least the largest such lo, L: every key >= L of every slice
//     lies in that slice's stored range.
//  2. topk_fine_emit_kernel: each slice block of the row sums the stored
//     histograms over 1024 keys at a time from the row's largest key down
//     until the rank k is reached, which fixes K*, the number of keys above it
//     and -- from the part of the sums over the slices before its own -- the
//     slice's output offset and the K*-ties already taken; then the slice's keys
//     above K* and the K*-ties the row still needs, lowest index first, are
//     written in ascending entry order.
// Rows run in groups of at most TKF_MAX_SLICES / P (P slices per row) per
// launch pair, which bounds the workspace: per slice a 16-byte header and a
// 128 KB histogram addressed by key (only [lo, hi] is written and read).
constexpr int TKF_THREADS = 512;
constexpr int TKF_SLICE = 16 * TKF_THREADS;   // entries per slice block
constexpr int TKF_KEYS = 1 << 16;             // bf16 keys
constexpr int TKF_MAX_SLICES = 1024;          // slices per launch pair
constexpr int TKF_NW = TKF_THREADS / 64;      // waves per block
constexpr int TKF_GPT = TKF_KEYS / 64 / TKF_THREADS;  // 64-key groups per thread
static_assert(TKF_GPT * TKF_THREADS * 64 == TKF_KEYS && TKF_NW <= 16, "block shape");
static_assert(TKF_MAX_SLICES % TKF_THREADS == 0, "whole header rounds");

struct TkfSlice {
  int lo, hi, count, pad;
};

static size_t tkf_hdr_bytes(int64_t slices) {
  return (size_t)((slices * (int64_t)sizeof(TkfSlice) + 255) / 256 * 256);
}

// exclusive scan over the TKF_THREADS threads of a block with one barrier;
// `ws` (one int per wave) must not be written again before a later barrier
__device__ __forceinline__ int tkf_block_excl(int v, int* ws, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_sum(v);
  if (lane == 63) ws[wave] = incl;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < TKF_THREADS / 64; ++i) {
    const int y = ws[i];
    pre += i < wave ? y : 0;
    tot += y;
  }
  *total = tot;
  return incl - v + pre;
}

// two exclusive scans at once (one barrier); `ws` holds two ints per wave
__device__ __forceinline__ void tkf_block_excl2(int a, int b, int* ws, int* ex_a, int* ex_b,
                                                int* tot_a, int* tot_b) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ia = wave_incl_sum(a), ib = wave_incl_sum(b);
  if (lane == 63) {
    ws[2 * wave] = ia;
    ws[2 * wave + 1] = ib;
  }
  __syncthreads();
  int pa = 0, pb = 0, ta = 0, tb = 0;
#pragma unroll
  for (int i = 0; i < TKF_THREADS / 64; ++i) {
    const int ya = ws[2 * i], yb = ws[2 * i + 1];
    pa += i < wave ? ya : 0;
    pb += i < wave ? yb : 0;
    ta += ya;
    tb += yb;
  }
  *ex_a = ia - a + pa;
  *ex_b = ib - b + pb;
  *tot_a = ta;
  *tot_b = tb;
}

// the raw bf16 scores of entries [s0, s0 + 16) of a row of Nmax (0 past Nmax),
// as 8 words; tkf_keys turns them into keys where they are first needed, so
// the loads stay in flight across other requests.  Entries past the row's
// visible count are masked by the caller.
__device__ __forceinline__ void tkf_load_raw(const uint16_t* srow, int s0, int Nmax, int vec,
                                             u32x4* raw) {
  if (vec && s0 + 16 <= Nmax) {
    const u32x4* p = reinterpret_cast<const u32x4*>(srow + s0);
    raw[0] = p[0];
    raw[1] = p[1];
  } else {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t a = (s0 + 2 * i < Nmax) ? srow[s0 + 2 * i] : 0u;
      const uint32_t b = (s0 + 2 * i + 1 < Nmax) ? srow[s0 + 2 * i + 1] : 0u;
      w[i] = a | (b << 16);
    }
    raw[0] = u32x4{w[0], w[1], w[2], w[3]};
    raw[1] = u32x4{w[4], w[5], w[6], w[7]};
  }
}
__device__ __forceinline__ void tkf_keys(const u32x4* raw, uint32_t* key) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      key[8 * j + 2 * i] = bf16_key(raw[j][i] & 0xFFFFu);
      key[8 * j + 2 * i + 1] = bf16_key(raw[j][i] >> 16);
    }
}

// count of key kk in the packed LDS histogram
__device__ __forceinline__ int tkf_count(const uint32_t* h, int kk) {
  const uint32_t v = h[kk >> 1];
  return (int)((kk & 1) ? (v >> 16) : (v & 0xFFFFu));
}
// the 64 keys of group g (words 32 g .. 32 g + 31), read from word `rot`
// mod 32 on so that the lanes of a wave hit distinct banks
__device__ __forceinline__ int tkf_group_count(const uint32_t* h, int g, int rot) {
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const uint32_t v = h[32 * g + ((j + rot) & 31)];
    cnt += (int)(v & 0xFFFFu) + (int)(v >> 16);
  }
  return cnt;
}

__global__ __launch_bounds__(TKF_THREADS) void topk_fine_hist_kernel(
    const uint16_t* __restrict__ scores, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int row0, int Tq, int Nmax, int m, int k, int vec,
    int P, TkfSlice* __restrict__ hdr, uint16_t* __restrict__ hist) {
  // counters of keys 2w (low half) and 2w+1 (high half), all cleared
  __shared__ __align__(16) uint32_t h[TKF_KEYS / 2];
  __shared__ __align__(16) int red[2][TKF_THREADS / 64];
  __shared__ __align__(16) int scan_ws[TKF_THREADS / 64];
  __shared__ int sh_grp[2];  // group holding the k-th largest key, keys above it
  __shared__ int sh_lo;
  const int lr = blockIdx.x / P, p = blockIdx.x % P, tid = threadIdx.x, lane = tid & 63;
  const int row = row0 + lr;
  // the slice's keys are requested together with the row's visible count, and
  // the histogram is cleared while they are in flight
  const int s0 = p * TKF_SLICE + 16 * tid;
  u32x4 raw[2];
  tkf_load_raw(scores + (int64_t)row * Nmax, s0, Nmax, vec, raw);
  const int nv = row_visible(q_pos, n_entries, row, Tq, Nmax, m);
  if (nv <= k) return;  // the emit kernel pads such rows; nothing here is read
  const int cs = min(max(nv - p * TKF_SLICE, 0), TKF_SLICE);
  if (cs == 0) {
    if (tid == 0) hdr[blockIdx.x] = TkfSlice{1, 0, 0, 0};
    return;
  }
  u32x4* h4 = reinterpret_cast<u32x4*>(h);
#pragma unroll
  for (int j = 0; j < TKF_KEYS / 8 / TKF_THREADS; ++j)
    h4[tid + j * TKF_THREADS] = u32x4{0u, 0u, 0u, 0u};
  uint32_t key[16];
  tkf_keys(raw, key);
  int kmax = -1, kmin = TKF_KEYS;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (s0 + i < nv) {
      kmax = max(kmax, (int)key[i]);
      kmin = min(kmin, (int)key[i]);
    }
  kmax = wave_all_max(kmax);
  kmin = wave_all_min(kmin);
  if (lane == 0) {
    red[0][tid >> 6] = kmax;
    red[1][tid >> 6] = kmin;
  }
  __syncthreads();  // histogram cleared, wave extremes stored
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (s0 + i < nv) atomicAdd(&h[key[i] >> 1], 1u << ((key[i] & 1u) << 4));
  const int hi = wave_all_max(lane < TKF_NW ? red[0][lane] : -1);
  int lo = wave_all_min(lane < TKF_NW ? red[1][lane] : TKF_KEYS);
  const int w_hi = hi >> 1;
  __syncthreads();  // histogram complete
  if (cs >= k) {
    const int g_hi = hi >> 6, g_lo = lo >> 6;
    if (g_hi - g_lo < 64) {
      // one wave: lane j counts group g_hi - j, then the keys of the group found
      if (tid < 64) {
        const int g = g_hi - lane;
        const int cnt = g >= g_lo ? tkf_group_count(h, g, lane) : 0;
        const int incl = wave_incl_sum(cnt);
        const uint64_t hit = __ballot(incl - cnt < k && incl >= k);
        const int jg = (int)__builtin_ctzll(hit);
        const int gs = max(g_hi - jg, 0), above = __builtin_amdgcn_readlane(incl - cnt, jg & 63);
        const int kk = 64 * gs + 63 - lane;
        const int c = tkf_count(h, kk);
        const int incl2 = wave_incl_sum(c) + above;
        const uint64_t hit2 = __ballot(incl2 - c < k && incl2 >= k);
        if (lane == 0) sh_lo = 64 * gs + 63 - (int)__builtin_ctzll(hit2);
      }
    } else {
      // thread t counts groups g_hi - TKF_GPT t - j, j < TKF_GPT (descending;
      // the range spans at most 1024 groups)
      int gc[TKF_GPT], cnt = 0;
#pragma unroll
      for (int j = 0; j < TKF_GPT; ++j) {
        const int g = g_hi - TKF_GPT * tid - j;
        gc[j] = g >= g_lo ? tkf_group_count(h, g, tid + j) : 0;
        cnt += gc[j];
      }
      if (tid == 0) {
        sh_grp[0] = g_lo;
        sh_grp[1] = 0;
      }
      int total;
      const int excl = tkf_block_excl(cnt, scan_ws, &total);
      if (excl < k && excl + cnt >= k) {
        int acc = excl, j = 0;
        while (j + 1 < TKF_GPT && acc + gc[j] < k) acc += gc[j++];
        sh_grp[0] = g_hi - TKF_GPT * tid - j;
        sh_grp[1] = acc;
      }
      __syncthreads();
      if (tid < 64) {
        const int kk = 64 * sh_grp[0] + 63 - lane;
        const int c = tkf_count(h, kk);
        const int incl2 = wave_incl_sum(c) + sh_grp[1];
        const uint64_t hit2 = __ballot(incl2 - c < k && incl2 >= k);
        if (lane == 0) sh_lo = 64 * sh_grp[0] + 63 - (int)__builtin_ctzll(hit2);
      }
    }
    __syncthreads();
    lo = min(max(sh_lo, lo), hi);  // within the slice's keys in any case
  }
  if (tid == 0) hdr[blockIdx.x] = TkfSlice{lo, hi, cs, 0};
  uint32_t* dst = reinterpret_cast<uint32_t*>(hist + (int64_t)blockIdx.x * TKF_KEYS);
  for (int w = (lo >> 1) + tid; w <= w_hi; w += TKF_THREADS) dst[w] = h[w];
}

__global__ __launch_bounds__(TKF_THREADS) void topk_fine_emit_kernel(
    const uint16_t* __restrict__ scores, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int row0, int Tq, int Nmax, int m, int k, int vec,
    int P, const TkfSlice* __restrict__ hdr, const uint16_t* __restrict__ hist,
    int32_t* __restrict__ idx) {
  __shared__ TkfSlice sh[TKF_MAX_SLICES];
  __shared__ __align__(16) int red[2][TKF_THREADS / 64];
  __shared__ __align__(16) int ws_cb[2 * (TKF_THREADS / 64)];
  __shared__ __align__(16) int ws_e[TKF_THREADS / 64];
  __shared__ int res[4];  // K*, keys above K*, of them in earlier slices, K*-ties in earlier slices
  const int lr = blockIdx.x / P, p = blockIdx.x % P, tid = threadIdx.x, lane = tid & 63;
  const int row = row0 + lr;
  // this slice's keys and the row's slice headers are requested together with
  // the row's visible count; the keys stay in flight while K* is found
  const int slice0 = p * TKF_SLICE;
  const int s0 = slice0 + 16 * tid;
  u32x4 raw[2];
  tkf_load_raw(scores + (int64_t)row * Nmax, s0, Nmax, vec, raw);
  const TkfSlice* hr = hdr + (int64_t)lr * P;
  TkfSlice hd[TKF_MAX_SLICES / TKF_THREADS];
#pragma unroll
  for (int j = 0; j < TKF_MAX_SLICES / TKF_THREADS; ++j) {
    const int i = tid + j * TKF_THREADS;
    if (i < P) hd[j] = hr[i];
  }
  const int nv = row_visible(q_pos, n_entries, row, Tq, Nmax, m);
  int32_t* out = idx + (int64_t)row * k;
  if (nv <= k) {
    for (int i = p * TKF_THREADS + tid; i < k; i += P * TKF_THREADS) out[i] = i < nv ? i : -1;
    return;
  }
  if (slice0 >= nv) return;
  const int pv = (nv + TKF_SLICE - 1) / TKF_SLICE;  // slices holding visible entries
  int L = -1, H = -1;
#pragma unroll
  for (int j = 0; j < TKF_MAX_SLICES / TKF_THREADS; ++j) {
    const int i = tid + j * TKF_THREADS;
    if (i < pv) {
      const TkfSlice d = hd[j];
      sh[i] = d;
      if (d.count >= k) L = max(L, d.lo);
      H = max(H, d.hi);
    }
  }
  L = wave_all_max(L);
  H = wave_all_max(H);
  if (lane == 0) {
    red[0][tid >> 6] = L;
    red[1][tid >> 6] = H;
  }
  if (tid < 4) res[tid] = tid == 0 ? -1 : 0;
  __syncthreads();
  L = wave_all_max(lane < TKF_NW ? red[0][lane] : -1);
  H = wave_all_max(lane < TKF_NW ? red[1][lane] : -1);
  // rank k from the top: thread t takes key top - t; counts of all slices (c)
  // and of the slices before this one (cb)
  const uint16_t* hrow = hist + (int64_t)lr * P * TKF_KEYS;
  int carry = 0, carry_before = 0;
  for (int top = H; top >= L; top -= TKF_THREADS) {
    const int kx = top - tid;
    int c = 0, cb = 0;
    if (kx >= L) {
      for (int sb = 0; sb < pv; sb += 32) {
        // unconditional loads from stored bins (slice and key clamped into a
        // stored range), masked afterwards: all 32 are in flight at once
        uint32_t v[32];
        bool in[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const int sl = min(sb + j, pv - 1);
          const int lo = sh[sl].lo, hi = sh[sl].hi;
          in[j] = sb + j < pv && kx >= lo && kx <= hi;
          v[j] = hrow[(int64_t)sl * TKF_KEYS + min(max(kx, lo), hi)];
        }
#pragma unroll
        for (int j = 0; j < 32; ++j) v[j] = in[j] ? v[j] : 0u;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          c += (int)v[j];
          cb += sb + j < p ? (int)v[j] : 0;
        }
      }
    }
    int ex_c, ex_b, tot_c, tot_b;
    tkf_block_excl2(c, cb, ws_cb, &ex_c, &ex_b, &tot_c, &tot_b);
    ex_c += carry;
    ex_b += carry_before;
    if (kx >= L && ex_c < k && ex_c + c >= k) {
      res[0] = kx;
      res[1] = ex_c;
      res[2] = ex_b;
      res[3] = cb;
    }
    __syncthreads();
    if (res[0] >= 0) break;
    carry += tot_c;
    carry_before += tot_b;
  }
  const uint32_t kstar = (uint32_t)res[0];
  const int need_eq = k - res[1];
  // ordered write of this slice's selection at its offset
  uint32_t key[16];
  tkf_keys(raw, key);
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bool ok = s0 + i < nv;
    gt += (ok && key[i] > kstar) ? 1 : 0;
    eq += (ok && key[i] == kstar) ? 1 : 0;
  }
  int total;
  const int excl = tkf_block_excl(gt | (eq << 16), ws_e, &total);
  int gt_before = res[2] + (excl & 0xFFFF), eq_before = res[3] + (excl >> 16);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bool ok = s0 + i < nv;
    const bool g = ok && key[i] > kstar, e = ok && key[i] == kstar;
    if (g || (e && eq_before < need_eq)) {
      const int pos = gt_before + min(eq_before, need_eq);
      if (pos >= 0 && pos < k) out[pos] = s0 + i;
    }
    gt_before += g ? 1 : 0;
    eq_before += e ? 1 : 0;
  }
}

static bool topk_bf16_long(csa_dtype score_t, int Nmax, int k) {
  return score_t == CSA_BF16 && Nmax > 16 * 1024 && k <= TKF_SLICE &&
         (Nmax + TKF_SLICE - 1) / TKF_SLICE <= TKF_MAX_SLICES;
}

static bool topk_multiblock(int Nmax) { return Nmax > 16 * 1024; }

// rows per launch pair of the long bf16 path
static int tkf_group(int64_t rows, int P) {
  const int64_t g = TKF_MAX_SLICES / P;
  return (int)(rows < g ? rows : g);
}

size_t topk_workspace(int B, int Tq, int Nmax) {
  if (!topk_multiblock(Nmax)) return 0;
  const int64_t rows = (int64_t)B * Tq;
  const int64_t P = (Nmax + TKM_SLICE - 1) / TKM_SLICE;
  // the larger of the two long-row paths (per-digit slice histograms and
  // counts; bf16 keys: per-slice 16-bit histograms of one row group)
  const size_t multi = (size_t)(rows * 4 + rows * P * 2048 + rows * P * 2) * sizeof(int);
  const int64_t Pf = (Nmax + TKF_SLICE - 1) / TKF_SLICE;
  size_t fine = 0;
  if (Pf <= TKF_MAX_SLICES && rows > 0) {
    const int64_t slices = (int64_t)tkf_group(rows, (int)Pf) * Pf;
    fine = tkf_hdr_bytes(slices) + (size_t)slices * TKF_KEYS * sizeof(uint16_t);
  }
  return multi > fine ? multi : fine;
}

hipError_t launch_topk(const void* scores, csa_dtype score_t, const int32_t* q_pos,
                       const int32_t* n_entries, int B, int Tq, int Nmax, int m, int k,
                       int32_t* idx, void* ws, hipStream_t s) {
  const int rows = B * Tq;
  if (rows == 0) return hipSuccess;
  const bool bf = score_t == CSA_BF16;
  // whole 16-byte key loads need 16-byte aligned rows
  const int vec = ((uintptr_t)scores % 16 == 0) && (bf ? Nmax % 8 == 0 : Nmax % 4 == 0);
  if (topk_bf16_long(score_t, Nmax, k)) {
    const int P = (Nmax + TKF_SLICE - 1) / TKF_SLICE;
    const int G = tkf_group(rows, P);
    TkfSlice* hdr = reinterpret_cast<TkfSlice*>(ws);
    uint16_t* hist = reinterpret_cast<uint16_t*>((char*)ws + tkf_hdr_bytes((int64_t)G * P));
    for (int r0 = 0; r0 < rows; r0 += G) {
      const int g = rows - r0 < G ? rows - r0 : G;
      const dim3 grid((unsigned)(g * P)), t(TKF_THREADS);
      hipLaunchKernelGGL(topk_fine_hist_kernel, grid, t, 0, s, (const uint16_t*)scores, q_pos,
                         n_entries, r0, Tq, Nmax, m, k, vec, P, hdr, hist);
      hipLaunchKernelGGL(topk_fine_emit_kernel, grid, t, 0, s, (const uint16_t*)scores, q_pos,
                         n_entries, r0, Tq, Nmax, m, k, vec, P, (const TkfSlice*)hdr,
                         (const uint16_t*)hist, idx);
    }
    return hipGetLastError();
  }
  if (topk_multiblock(Nmax)) {
    const int P = (Nmax + TKM_SLICE - 1) / TKM_SLICE;
    TkRow* st = reinterpret_cast<TkRow*>(ws);
    int* hist = reinterpret_cast<int*>(ws) + (int64_t)rows * 4;
    int* cnt = hist + (int64_t)rows * P * 2048;
    const dim3 g((unsigned)((int64_t)rows * P)), t(TKM_THREADS);
    // digits: bf16 keys 8 + 8 bits, fp32 keys 11 + 11 + 10 bits
    int shift = bf ? 16 : 32, first = 1;
    while (shift > 0) {
      const int width = bf ? 8 : (shift == 32 || shift == 21 ? 11 : 10);
      shift -= width;
      if (bf)
        hipLaunchKernelGGL(topk_hist_kernel<true>, g, t, 0, s, scores, q_pos, n_entries, Tq, Nmax,
                           m, k, vec, P, shift, width, first ? nullptr : st, hist);
      else
        hipLaunchKernelGGL(topk_hist_kernel<false>, g, t, 0, s, scores, q_pos, n_entries, Tq, Nmax,
                           m, k, vec, P, shift, width, first ? nullptr : st, hist);
      hipLaunchKernelGGL(topk_reduce_kernel, dim3(rows), dim3(1024), 0, s, q_pos, n_entries, Tq,
                         Nmax, m, k, P, shift, width, first, st, hist);
      first = 0;
    }
    if (bf) {
      hipLaunchKernelGGL(topk_count_kernel<true>, g, t, 0, s, scores, q_pos, n_entries, Tq, Nmax,
                         m, k, vec, P, st, cnt);
      hipLaunchKernelGGL(topk_emit_kernel<true>, g, t, 0, s, scores, q_pos, n_entries, Tq, Nmax,
                         m, k, vec, P, st, cnt, idx);
    } else {
      hipLaunchKernelGGL(topk_count_kernel<false>, g, t, 0, s, scores, q_pos, n_entries, Tq, Nmax,
                         m, k, vec, P, st, cnt);
      hipLaunchKernelGGL(topk_emit_kernel<false>, g, t, 0, s, scores, q_pos, n_entries, Tq, Nmax,
                         m, k, vec, P, st, cnt, idx);
    }
    return hipGetLastError();
  }
  // one block per row, 16 keys per thread (counts stay below 2^16 for the packed scan)
  int threads = 64;  // the smallest power of two >= Nmax / 16, at least one wave
  while (threads * 16 < Nmax) threads *= 2;
  const size_t cand_bytes = (size_t)(16 * threads < TK_CAND_CAP ? 16 * threads : TK_CAND_CAP) * sizeof(uint32_t);
  // more rows than compute units: occupancy counts more than a row's latency
  // (the selection is exact either way)
  if (bf)
    hipLaunchKernelGGL((topk_kernel<true, 13>), dim3(rows), dim3(threads), cand_bytes, s, scores,
                       q_pos, n_entries, Tq, Nmax, m, k, vec, idx);
  else if (rows > 256)
    hipLaunchKernelGGL(topk_many_kernel, dim3(rows), dim3(threads), cand_bytes, s, scores, q_pos,
                       n_entries, Tq, Nmax, m, k, vec, idx);
  else
    hipLaunchKernelGGL((topk_kernel<false, 13>), dim3(rows), dim3(threads), cand_bytes, s, scores,
                       q_pos, n_entries, Tq, Nmax, m, k, vec, idx);
  return hipGetLastError();
}

}  // namespace csa
