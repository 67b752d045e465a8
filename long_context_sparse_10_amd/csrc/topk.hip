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
// block-wide scan.  Longer rows (few decode rows over 2^18 entries) spread over
// many blocks per row: per-block digit histograms, a per-row reduction that
// fixes the digit, and after the last digit per-block counts and an ordered
// emit at each block's offset.
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

// exclusive block scan of one int per thread; *total gets the block sum.
// `ws` is LDS of >= 16 ints.  Every thread of the block must call.
__device__ __forceinline__ int block_scan_excl(int v, int* ws, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(x, o);
    if (lane >= o) x += t;
  }
  if (lane == 63) ws[wave] = x;
  __syncthreads();
  int pre = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const int y = ws[i];
    pre += (i < wave) ? y : 0;
    tot += y;
  }
  __syncthreads();
  *total = tot;
  return x - v + pre;
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

// exclusive prefix of one int per lane within the wave; *total gets the wave sum
__device__ __forceinline__ int wave_scan_excl(int v, int* total) {
  const int lane = threadIdx.x & 63;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(x, o);
    if (lane >= o) x += t;
  }
  *total = __shfl(x, 63);
  return x - v;
}

// candidates compacted for the last digits (more go the block-wide way): a
// small buffer keeps more rows resident per CU when many short rows run
constexpr int TK_CAND_CAP = 2048;

// W1: width of the first digit of fp32 keys (13, or 12 when many rows share the
// GPU: a 16 KB histogram lets four 512-thread blocks reside per CU instead of
// three).  bf16 keys take 10 then 6 bits.
template <bool BF16, int W1>
__global__ __launch_bounds__(1024) void topk_kernel(const void* __restrict__ scores,
                                                    const int32_t* __restrict__ q_pos,
                                                    const int32_t* __restrict__ n_entries, int Tq,
                                                    int Nmax, int m, int k, int vec,
                                                    int32_t* __restrict__ idx) {
  __shared__ int hist[BF16 ? 1024 : (1 << W1)];
  extern __shared__ uint32_t cand[];  // [min(16 * blockDim, TK_CAND_CAP)]: keys sharing the k-th's first digit
  __shared__ int scan_ws[16];
  __shared__ uint32_t sh_digit;
  __shared__ int sh_above, sh_ncand;
  const int row = blockIdx.x, b = row / Tq;
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63;
  const int cap = min(16 * nt, TK_CAND_CAP);
  const int nv = min(min(n_entries[b], Nmax), (q_pos[row] + 1) / m);
  int32_t* out = idx + (int64_t)row * k;
  const void* srow = BF16 ? (const void*)((const uint16_t*)scores + (int64_t)row * Nmax)
                          : (const void*)((const uint32_t*)scores + (int64_t)row * Nmax);
  if (nv <= k) {
    for (int i = tid; i < k; i += nt) out[i] = i < nv ? i : -1;
    return;
  }
  // ---- keys in registers: thread t owns entries [16 t, 16 t + 16)
  uint32_t key[16];
  const int s0 = tid * 16;
  if (vec) {
    // a wave whose 1,024 entries all lie past the visible count loads nothing
    // (its keys are masked everywhere); in a causal prefill that is about half
    if (__builtin_amdgcn_readfirstlane(tid >> 6) * 1024 < nv) {
      load_keys16<BF16>(srow, s0, nv, Nmax, key);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) key[i] = 0u;
    }
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
    // ---- remaining digits over the candidates by wave 0 alone (no block barriers):
    // fp32 keys 10 + 9 (W1 13) or 10 + 10 bits (W1 12), bf16 keys 6 bits (5..0)
    uint32_t prefix = d1 << SH1, pmask = ~0u << SH1;
    int shift = SH1;
    while (shift > 0) {
      const int width = BF16 ? 6 : min(shift, 10);
      shift -= width;
      const int nbins = 1 << width;
      const uint32_t dmask = (uint32_t)nbins - 1u;
      for (int i = lane; i < nbins; i += 64) hist[i] = 0;
      __builtin_amdgcn_wave_barrier();
      for (int i = lane; i < nc; i += 64) {
        const uint32_t kk = cand[i];
        if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & dmask], 1);
      }
      __builtin_amdgcn_wave_barrier();
      find_digit(hist, nbins, remaining, &sh_digit, &sh_above);
      __builtin_amdgcn_wave_barrier();
      const uint32_t dg = __shfl(sh_digit, 0);
      remaining -= __shfl(sh_above, 0);
      prefix |= dg << shift;
      pmask |= dmask << shift;
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

static bool topk_multiblock(int Nmax) { return Nmax > 16 * 1024; }

size_t topk_workspace(int B, int Tq, int Nmax) {
  if (!topk_multiblock(Nmax)) return 0;
  const int64_t rows = (int64_t)B * Tq;
  const int64_t P = (Nmax + TKM_SLICE - 1) / TKM_SLICE;
  return (size_t)(rows * 4 + rows * P * 2048 + rows * P * 2) * sizeof(int);
}

hipError_t launch_topk(const void* scores, csa_dtype score_t, const int32_t* q_pos,
                       const int32_t* n_entries, int B, int Tq, int Nmax, int m, int k,
                       int32_t* idx, void* ws, hipStream_t s) {
  const int rows = B * Tq;
  if (rows == 0) return hipSuccess;
  const bool bf = score_t == CSA_BF16;
  // whole 16-byte key loads need 16-byte aligned rows
  const int vec = ((uintptr_t)scores % 16 == 0) && (bf ? Nmax % 8 == 0 : Nmax % 4 == 0);
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
    hipLaunchKernelGGL((topk_kernel<false, 12>), dim3(rows), dim3(threads), cand_bytes, s, scores,
                       q_pos, n_entries, Tq, Nmax, m, k, vec, idx);
  else
    hipLaunchKernelGGL((topk_kernel<false, 13>), dim3(rows), dim3(threads), cand_bytes, s, scores,
                       q_pos, n_entries, Tq, Nmax, m, k, vec, idx);
  return hipGetLastError();
}

}  // namespace csa
