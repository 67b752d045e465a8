// Lightning indexer (Evidence Ledger Eqs 13-17; shuhuayu section 03 score):
//   score(t, s) = sum_h w[t, h] * ReLU(qI[t, h] . kI[s])   for s < N(q_t).
//
// Hot shape (cI = 128, nI = 64, bf16 or MXFP4): the q.k contraction runs on
// the matrix cores with the 64 heads as the M dimension (four 16-row tiles)
// and 16 entries per group as N, K = 128.  Each lane then holds one entry
// column and 4 head rows of each tile, so the ReLU-weighted head reduction is
// 16 in-register FMAs plus two exchanges across the lane groups.  Index keys
// stream straight from HBM into MFMA operand registers: the K order inside an
// MFMA is free, so the lanes of an entry take contiguous bytes of its row and
// the query fragments use the same permutation.  MXFP4 keys and queries go to the
// block-scaled fp4 MFMA as stored (E2M1 codes plus e8m0 scales); products of
// E2M1 values times powers of two are exact and accumulate in fp32.
#include "common.hpp"
#include "internal.hpp"

namespace csa {

// ------------------------------------------------------------------ generic
// any nI, cI; one thread per entry, the query (dequantised) staged in LDS
__device__ __forceinline__ float load_index_elem(const uint8_t* row, const uint8_t* scales,
                                                 csa_dtype t, int j) {
  if (t == CSA_F32) return reinterpret_cast<const float*>(row)[j];
  if (t == CSA_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[j]);
  const uint32_t byte = row[j >> 1];
  const uint32_t code = (j & 1) ? (byte >> 4) : (byte & 15u);
  return e2m1_to_f32(code) * exp2i((int)scales[j >> 5] - 127);
}

// ReLU of a matrix-core result in one v_med3_f32: med3(x, 0, FLT_MAX) = max(x, 0)
// for finite x, without the NaN-quieting max(x, x) the compiler puts in front of
// fmaxf on values it cannot prove canonical (it doubled the epilogue's VALU work)
__device__ __forceinline__ float relu_mfma(float x) {
  return __builtin_amdgcn_fmed3f(x, 0.f, 3.402823466e38f);
}

__global__ __launch_bounds__(256) void indexer_generic_kernel(
    const uint8_t* __restrict__ qI, const uint8_t* __restrict__ qI_scale, csa_dtype t,
    const float* __restrict__ w, const uint8_t* __restrict__ kI, const uint8_t* __restrict__ kI_scale,
    const int32_t* __restrict__ q_pos, const int32_t* __restrict__ n_entries, int Tq, int nI,
    int cI, int Nmax, int m, void* __restrict__ scores, int score_bf16, PageMap pg) {
  extern __shared__ float sq[];  // [nI * cI] query, then [nI] weights
  const int tiles = (Nmax + blockDim.x - 1) / blockDim.x;
  const int row = blockIdx.x / tiles, tile = blockIdx.x % tiles, b = row / Tq;
  const int nv = min(min(n_entries[b], Nmax), (q_pos[row] + 1) / m);
  if (tile * (int)blockDim.x >= nv) return;
  const int64_t qrb = row_bytes(t, cI, 0);
  for (int i = threadIdx.x; i < nI * cI; i += blockDim.x) {
    const int h = i / cI, j = i % cI;
    const int64_t qr = (int64_t)row * nI + h;
    sq[i] = load_index_elem(qI + qr * qrb, qI_scale ? qI_scale + qr * (cI / 32) : nullptr, t, j);
  }
  for (int h = threadIdx.x; h < nI; h += blockDim.x) sq[nI * cI + h] = w[(int64_t)row * nI + h];
  __syncthreads();
  const int s = tile * blockDim.x + threadIdx.x;
  if (s >= nv) return;
  const uint8_t* krow = kI + pg.off(b, s, Nmax, qrb);
  const uint8_t* ksc = kI_scale ? kI_scale + pg.off(b, s, Nmax, cI / 32) : nullptr;
  float score = 0.f;
  for (int h = 0; h < nI; ++h) {
    float dot = 0.f;
    for (int j = 0; j < cI; ++j) dot = fmaf(sq[h * cI + j], load_index_elem(krow, ksc, t, j), dot);
    score = fmaf(sq[nI * cI + h], fmaxf(dot, 0.f), score);
  }
  const int64_t o = (int64_t)row * Nmax + s;
  if (score_bf16)
    reinterpret_cast<uint16_t*>(scores)[o] = (uint16_t)f32_to_bf16(score);
  else
    reinterpret_cast<float*>(scores)[o] = score;
}

// ------------------------------------------------------------------ MFMA (nI 64, cI 128)
constexpr int IDX_WAVES = 4;

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i32x8 widen(u32x4 v) {
  return i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
}

// Head sums of two 16-entry groups.  part0 / part1 are this lane's partial
// sums (heads 16mt + 4kg + r) for group A / B; the four 16-lane rows (kg) are
// added with two lane swaps on the VALU.  The 16-lane swap exchanges odd rows
// of the first operand with even rows of the second: rows become (A: kg 0+1,
// B: kg 0+1, A: kg 2+3, B: kg 2+3); the 32-lane swap then adds the upper half
// to the lower.  Lane l < 32 returns the score of entry l of the 32 (A's 16,
// then B's).
__device__ __forceinline__ float head_sum_pair(float part0, float part1) {
  const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(part0), __float_as_uint(part1),
                                                 false, false);
  const float t = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false,
                                                 false);
  return __uint_as_float(y[0]) + __uint_as_float(y[1]);
}

// One block = 4 waves over a contiguous entry range of one query row.  The
// contraction uses 16x16 matrix-core tiles: 4 tiles of 16 heads (M) by 16
// entries (N).  Lane (col, kg) = (lane % 16, lane / 16) holds entry col; the
// four lanes of an entry read adjacent 16-byte pieces of its row, so every
// load instruction covers 16 rows in 64-byte contiguous runs.
//  * bf16: v_mfma_f32_16x16x32_bf16, step ks covers row bytes 64ks .. 64ks+63
//    (lane kg: dims 32ks + 8kg .. +7), K = 128 in 4 steps.
//  * MXFP4: v_mfma_scale_f32_16x16x128_f8f6f4, one instruction per tile: lane
//    kg holds code bytes 16kg .. 16kg+15 (dims 32kg .. 32kg+31), exactly the
//    32-element block whose e8m0 scale the matrix core applies.
// A wave scores G groups of 16 entries per step (bf16 G = 2, MXFP4 G = 4),
// reduces the head sum of two groups at a time across its four lane rows, and
// keeps a ring of three steps of raw key bytes in registers: two in flight
// while the third is scored.
template <bool MX>
__global__ __launch_bounds__(IDX_WAVES * 64, MX ? 4 : 2) void indexer_mfma_kernel(
    const uint8_t* __restrict__ qI, const uint8_t* __restrict__ qI_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ kI,
    const uint8_t* __restrict__ kI_scale, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int Nmax, int m, int ent_per_block,
    void* __restrict__ scores, int score_bf16, PageMap pg) {
  constexpr int G = MX ? 4 : 2;
  constexpr int64_t RB = MX ? 64 : 256;  // key row bytes
  extern __shared__ __attribute__((aligned(16))) uint32_t sbuf[];  // the block's scores
  const int tiles = (Nmax + ent_per_block - 1) / ent_per_block;
  const int row = blockIdx.x / tiles, b = row / Tq;
  // the wave index as a scalar: the step loop below is then uniform control flow
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kg = lane >> 4, col = lane & 15;
  const int e0 = (blockIdx.x % tiles) * ent_per_block;
  // dense rows: the first two steps are fetched before the visible-entry
  // count arrives (rows up to the block's end or Nmax are in bounds; scores
  // past the count are not written).  Paged rows wait for the count.
  int e1 = min(e0 + ent_per_block, Nmax);

  struct Raw {
    u32x4 v[MX ? G : 4 * G];
    uint32_t sc[MX ? G : 1];
  };
  auto fetch = [&](int base, Raw& r) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int n = base + 16 * g + col;
      // key row and scale row offsets: dense rows b * Nmax + n, or slot n % 2^shift of
      // the page holding entry n (the scales share the key rows' pages)
      int64_t ko, so;
      if (pg.paged()) {
        // a 16-entry group lies in one page (pages hold >= 16 entries, groups
        // start at multiples of 16): one wave-uniform page id per group, a
        // scalar load that does not wait behind the key loads in flight.
        // Lanes past the visible range read the group's first row (or e0's).
        const int gs = __builtin_amdgcn_readfirstlane(base) + 16 * g;
        const int ge = gs < e1 ? gs : e0;
        const int nn = n < e1 ? n : ge;
        // the page table does not change during the kernel: read it through
        // the constant address space, a scalar load at a uniform address
        const __attribute__((address_space(4))) int32_t* tab =
            (const __attribute__((address_space(4))) int32_t*)pg.table;
        const int64_t pb = (int64_t)tab[(int64_t)b * pg.max_blocks + (ge >> pg.shift)] * pg.page_bytes;
        const int sl = nn & ((1 << pg.shift) - 1);
        ko = pb + (int64_t)sl * RB;
        so = pb + (int64_t)sl * 4;
      } else {
        const int64_t kr = (int64_t)b * Nmax + (n < e1 ? n : e0);
        ko = kr * RB;
        so = kr * 4;
      }
      if (!MX) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          r.v[4 * g + ks] = *reinterpret_cast<const u32x4*>(kI + ko + 64 * ks + 16 * kg);
      } else {
        r.v[g] = *reinterpret_cast<const u32x4*>(kI + ko + 16 * kg);
        r.sc[g] = *reinterpret_cast<const uint32_t*>(kI_scale + so);
      }
    }
  };
  // query fragments of head 16*mt + col in the keys' K order (loaded before
  // the keys, so that their first use waits for none of the key loads)
  bf16x8 afr[4][MX ? 1 : 4];
  u32x4 aq[4];
  int asc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int64_t qr = (int64_t)row * 64 + 16 * mt + col;
    if (!MX) {
#pragma unroll
      for (int ks = 0; ks < (MX ? 1 : 4); ++ks)
        afr[mt][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qI + qr * 256 + 64 * ks + 16 * kg));
    } else {
      aq[mt] = *reinterpret_cast<const u32x4*>(qI + qr * 64 + 16 * kg);
      asc[mt] = (int)(*reinterpret_cast<const uint32_t*>(qI_scale + qr * 4) >> (8 * kg));
    }
  }
  // weights of the head rows this lane's accumulators hold: register r of
  // tile mt is head 16*mt + 4*kg + r
  float wr[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) wr[mt][r] = w[(int64_t)row * 64 + 16 * mt + 4 * kg + r];

  // Every fetch below is unconditional (steps past the range read in-bounds
  // rows and are not scored): with a fixed number of loads per step, the
  // compiler's in-order load counts let a step's keys be used while the two
  // later steps are still in flight.  A fetch under a condition made it
  // assume the later steps might be absent and wait for all loads instead.
  constexpr int STEP = IDX_WAVES * 16 * G;
  int base = e0 + wave * 16 * G;
  Raw r0, r1, r2;
  if (!pg.paged()) {
    fetch(base, r0);
    fetch(base + STEP, r1);
  }
  const int nv = min(min(n_entries[b], Nmax), (q_pos[row] + 1) / m);
  if (e0 >= nv) return;
  e1 = min(e1, nv);
  if (pg.paged()) {
    fetch(base, r0);
    fetch(base + STEP, r1);
  }

  auto process = [&](const Raw& r, int base) {
#pragma unroll
    for (int gp = 0; gp < G; gp += 2) {
      float part[2];  // this lane's share (heads 16mt + 4kg + r) of groups gp, gp + 1
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int g = gp + h;
        f32x4 acc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!MX) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 bk = __builtin_bit_cast(bf16x8, r.v[4 * g + ks]);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
              acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[mt][MX ? 0 : ks], bk, acc[mt], 0, 0, 0);
          }
        } else {
          const i32x8 bk = widen(r.v[g]);
          const int bs = (int)(r.sc[MX ? g : 0] >> (8 * kg));
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(widen(aq[mt]), bk, acc[mt], 4, 4, 0, asc[mt], 0, bs);
        }
        float sc = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) sc = fmaf(wr[mt][q], relu_mfma(acc[mt][q]), sc);
        part[h] = sc;
      }
      // lane l < 32: the score of entry 16 gp + l
      const float sc = head_sum_pair(part[0], part[1]);
      const int n = base + 16 * gp + lane;
      if (lane < 32 && n < e1) {
        if (score_bf16)
          reinterpret_cast<uint16_t*>(sbuf)[n - e0] = (uint16_t)f32_to_bf16(sc);
        else
          sbuf[n - e0] = __float_as_uint(sc);
      }
    }
  };
  // every load so far has landed (the first two key steps as well: the first
  // is needed now and the second left right after it).  With nothing in
  // flight at its head, the loop's in-order counts cover key steps alone and
  // each step waits only for its own keys; a partial wait here left the
  // compiler assuming older loads in flight, and it drained the next step too.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  // whole triples of steps, then the last one or two (already in r0, r1);
  // the loop has no other exit, so no step's loads are thought pending at
  // its head
  for (; base + 2 * STEP < e1; base += 3 * STEP) {
    fetch(base + 2 * STEP, r2);
    process(r0, base);
    fetch(base + 3 * STEP, r0);
    process(r1, base + STEP);
    fetch(base + 4 * STEP, r1);
    process(r2, base + 2 * STEP);
  }
  if (base < e1) process(r0, base);
  if (base + STEP < e1) process(r1, base + STEP);
  // the block's scores leave once, after the key stream: a store issued
  // between key loads would hold up the in-order wait for the next key step
  __syncthreads();
  const int len = e1 - e0;
  const int64_t o0 = (int64_t)row * Nmax + e0;
  const int per16 = score_bf16 ? 8 : 4;  // scores per 16 bytes
  uint8_t* dst = reinterpret_cast<uint8_t*>(scores) + o0 * (score_bf16 ? 2 : 4);
  const int nvec = ((uintptr_t)dst & 15) == 0 ? len / per16 : 0;
  for (int i = threadIdx.x; i < nvec; i += IDX_WAVES * 64)
    reinterpret_cast<u32x4*>(dst)[i] = reinterpret_cast<const u32x4*>(sbuf)[i];
  for (int i = nvec * per16 + threadIdx.x; i < len; i += IDX_WAVES * 64) {
    if (score_bf16)
      reinterpret_cast<uint16_t*>(dst)[i] = reinterpret_cast<const uint16_t*>(sbuf)[i];
    else
      reinterpret_cast<uint32_t*>(dst)[i] = sbuf[i];
  }
}

// ------------------------------------------------------------------ many query rows
// Prefill shape (bf16, nI 64, cI 128, many query rows per sequence): one
// block scores IR_ROWS consecutive query rows of a sequence, one wave per row
// with its query fragments in registers.  The rows share every index key, so
// keys pass through LDS once per block in 128-entry chunks (double buffered,
// staged through registers one chunk ahead) and each wave reads them from
// there.  Blocks run from the last (longest) rows backwards.
constexpr int IR_ROWS = 16;  // query rows per block (measured: 4 -> 2.44 ms, 16 -> 2.06 ms at 32K)
constexpr int IR_CH = 128;  // entries per key chunk
constexpr int IR_LD = 136;  // LDS row stride in bf16 (272 B: 16 rows at one column hit 64 banks)

template <int R>  // query rows per block, one wave each
__global__ __launch_bounds__(64 * R) void indexer_rows_kernel(
    const uint8_t* __restrict__ qI, const float* __restrict__ w, const uint8_t* __restrict__ kI,
    const int32_t* __restrict__ q_pos, const int32_t* __restrict__ n_entries, int B, int Tq,
    int Nmax, int m, void* __restrict__ scores, int score_bf16) {
  __shared__ __attribute__((aligned(16))) uint16_t K[2][IR_CH][IR_LD];
  constexpr int NT = 64 * R;
  const int gps = (Tq + R - 1) / R;
  const int grp = (int)gridDim.x - 1 - (int)blockIdx.x;
  const int b = grp / gps, r0 = (grp % gps) * R;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 4, col = lane & 15;
  const int nent = min(n_entries[b], Nmax);
  int nv_max = 0;
#pragma unroll
  for (int j = 0; j < R; ++j)
    if (r0 + j < Tq) nv_max = max(nv_max, min(nent, (q_pos[b * Tq + r0 + j] + 1) / m));
  if (nv_max == 0) return;
  const bool has_row = r0 + wave < Tq;
  const int row = b * Tq + r0 + (has_row ? wave : 0);
  const int nv = has_row ? min(nent, (q_pos[row] + 1) / m) : 0;

  bf16x8 afr[4][4];
  float wr[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int64_t qr = (int64_t)row * 64 + 16 * mt + col;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      afr[mt][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qI + qr * 256 + 64 * ks + 16 * kg));
#pragma unroll
    for (int r = 0; r < 4; ++r) wr[mt][r] = w[(int64_t)row * 64 + 16 * mt + 4 * kg + r];
  }
  // chunk staging: thread t moves bytes 16 (t % 16) of entries t / 16 + (NT / 16) i
  constexpr int NI = IR_CH * 16 / NT;  // 16-byte pieces per thread per chunk
  const uint8_t* kb = kI + (int64_t)b * Nmax * 256;
  const int nch = (nv_max + IR_CH - 1) / IR_CH;
  u32x4 st[NI];
  auto fetch = [&](int c) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int n = c * IR_CH + tid / 16 + (NT / 16) * i;
      st[i] = *reinterpret_cast<const u32x4*>(kb + (int64_t)(n < nv_max ? n : 0) * 256 + 16 * (tid % 16));
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      *reinterpret_cast<u32x4*>(&K[buf][tid / 16 + (NT / 16) * i][8 * (tid % 16)]) = st[i];
  };
  fetch(0);
  commit(0);
  if (nch > 1) fetch(1);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    // two 16-entry groups per step (entries past the row are staged copies of
    // entry 0: scored, never stored)
    for (int gi = 0; gi < IR_CH / 16; gi += 2) {
      const int n0 = c * IR_CH + 16 * gi;
      if (n0 >= nv) break;
      float part[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 acc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 bk =
              *reinterpret_cast<const bf16x8*>(&K[buf][16 * (gi + h) + col][32 * ks + 8 * kg]);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[mt][ks], bk, acc[mt], 0, 0, 0);
        }
        float sc = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) sc = fmaf(wr[mt][q], relu_mfma(acc[mt][q]), sc);
        part[h] = sc;
      }
      const float sc = head_sum_pair(part[0], part[1]);
      const int n = n0 + lane;
      if (lane < 32 && n < nv) {
        const int64_t o = (int64_t)row * Nmax + n;
        if (score_bf16)
          reinterpret_cast<uint16_t*>(scores)[o] = (uint16_t)f32_to_bf16(sc);
        else
          reinterpret_cast<float*>(scores)[o] = sc;
      }
    }
    if (c + 1 < nch) {
      commit((c + 1) & 1);
      if (c + 2 < nch) fetch(c + 2);
    }
    __syncthreads();
  }
}

// MXFP4 form of indexer_rows_kernel: 256-entry chunks of E2M1 codes (80-byte
// LDS rows, conflict-free for 16 lanes at one column) plus their e8m0 scale
// dwords; each 16-entry group is 4 block-scaled fp4 MFMAs (one per head tile).
constexpr int IRX_CH = 256;  // entries per key chunk
constexpr int IRX_LD = 80;   // LDS bytes per staged row (64 bytes of codes)

template <int R>
__global__ __launch_bounds__(64 * R) void indexer_rows_mx_kernel(
    const uint8_t* __restrict__ qI, const uint8_t* __restrict__ qI_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ kI,
    const uint8_t* __restrict__ kI_scale, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int B, int Tq, int Nmax, int m,
    void* __restrict__ scores, int score_bf16) {
  static_assert(64 * R == 4 * IRX_CH, "one 16-byte piece of codes per thread per chunk");
  __shared__ __attribute__((aligned(16))) uint8_t Kc[2][IRX_CH][IRX_LD];
  __shared__ uint32_t Ks[2][IRX_CH];
  const int gps = (Tq + R - 1) / R;
  const int grp = (int)gridDim.x - 1 - (int)blockIdx.x;
  const int b = grp / gps, r0 = (grp % gps) * R;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 4, col = lane & 15;
  const int nent = min(n_entries[b], Nmax);
  int nv_max = 0;
#pragma unroll
  for (int j = 0; j < R; ++j)
    if (r0 + j < Tq) nv_max = max(nv_max, min(nent, (q_pos[b * Tq + r0 + j] + 1) / m));
  if (nv_max == 0) return;
  const bool has_row = r0 + wave < Tq;
  const int row = b * Tq + r0 + (has_row ? wave : 0);
  const int nv = has_row ? min(nent, (q_pos[row] + 1) / m) : 0;

  // query fragments of head 16 mt + col: codes of dims 32 kg .. 32 kg + 31 and
  // their scale (in byte 0)
  u32x4 aq[4];
  int asc[4];
  float wr[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int64_t qr = (int64_t)row * 64 + 16 * mt + col;
    aq[mt] = *reinterpret_cast<const u32x4*>(qI + qr * 64 + 16 * kg);
    asc[mt] = (int)(*reinterpret_cast<const uint32_t*>(qI_scale + qr * 4) >> (8 * kg));
#pragma unroll
    for (int r = 0; r < 4; ++r) wr[mt][r] = w[(int64_t)row * 64 + 16 * mt + 4 * kg + r];
  }
  // staging: thread t moves code bytes 16 (t % 4) of entry t / 4; threads below
  // IRX_CH also move entry t's scale dword
  const uint8_t* kb = kI + (int64_t)b * Nmax * 64;
  const uint32_t* ksb = reinterpret_cast<const uint32_t*>(kI_scale) + (int64_t)b * Nmax;
  const int nch = (nv_max + IRX_CH - 1) / IRX_CH;
  u32x4 st;
  uint32_t ss = 0u;
  auto fetch = [&](int c) {
    const int n = c * IRX_CH + tid / 4;
    st = *reinterpret_cast<const u32x4*>(kb + (int64_t)(n < nv_max ? n : 0) * 64 + 16 * (tid % 4));
    if (tid < IRX_CH) {
      const int ns = c * IRX_CH + tid;
      ss = ksb[ns < nv_max ? ns : 0];
    }
  };
  auto commit = [&](int buf) {
    *reinterpret_cast<u32x4*>(&Kc[buf][tid / 4][16 * (tid % 4)]) = st;
    if (tid < IRX_CH) Ks[buf][tid] = ss;
  };
  fetch(0);
  commit(0);
  if (nch > 1) fetch(1);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    // two 16-entry groups per step (entries past the row are staged copies of
    // entry 0: scored, never stored)
    for (int gi = 0; gi < IRX_CH / 16; gi += 2) {
      const int n0 = c * IRX_CH + 16 * gi;
      if (n0 >= nv) break;
      float part[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const i32x8 bk =
            widen(*reinterpret_cast<const u32x4*>(&Kc[buf][16 * (gi + h) + col][16 * kg]));
        const int bs = (int)(Ks[buf][16 * (gi + h) + col] >> (8 * kg));
        f32x4 acc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              widen(aq[mt]), bk, f32x4{0.f, 0.f, 0.f, 0.f}, 4, 4, 0, asc[mt], 0, bs);
        float sc = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) sc = fmaf(wr[mt][q], relu_mfma(acc[mt][q]), sc);
        part[h] = sc;
      }
      const float sc = head_sum_pair(part[0], part[1]);
      const int n = n0 + lane;
      if (lane < 32 && n < nv) {
        const int64_t o = (int64_t)row * Nmax + n;
        if (score_bf16)
          reinterpret_cast<uint16_t*>(scores)[o] = (uint16_t)f32_to_bf16(sc);
        else
          reinterpret_cast<float*>(scores)[o] = sc;
      }
    }
    if (c + 1 < nch) {
      commit((c + 1) & 1);
      if (c + 2 < nch) fetch(c + 2);
    }
    __syncthreads();
  }
}

hipError_t launch_indexer(const void* qI, const uint8_t* qI_scale, csa_dtype in_t, const float* w,
                          const void* kI, const uint8_t* kI_scale, const int32_t* q_pos,
                          const int32_t* n_entries, int B, int Tq, int nI, int cI, int Nmax,
                          int m, void* scores, csa_dtype score_t, hipStream_t s,
                          const PageMap& pg) {
  const int rows = B * Tq;
  if (rows == 0 || Nmax == 0) return hipSuccess;
  const int sbf = score_t == CSA_BF16;
  // the many-query-row kernels stage dense key chunks; paged keys take the
  // per-row kernel
  if (in_t == CSA_BF16 && nI == 64 && cI == 128 && Tq >= IR_ROWS && !pg.paged()) {
    const int64_t groups = (int64_t)B * ((Tq + IR_ROWS - 1) / IR_ROWS);
    hipLaunchKernelGGL(indexer_rows_kernel<IR_ROWS>, dim3((unsigned)groups), dim3(64 * IR_ROWS), 0,
                       s, (const uint8_t*)qI, w, (const uint8_t*)kI, q_pos, n_entries, B, Tq,
                       Nmax, m, scores, sbf);
  } else if (in_t == CSA_MXFP4 && nI == 64 && cI == 128 && Tq >= IR_ROWS && !pg.paged()) {
    const int64_t groups = (int64_t)B * ((Tq + IR_ROWS - 1) / IR_ROWS);
    hipLaunchKernelGGL(indexer_rows_mx_kernel<IR_ROWS>, dim3((unsigned)groups),
                       dim3(64 * IR_ROWS), 0, s, (const uint8_t*)qI, qI_scale, w,
                       (const uint8_t*)kI, kI_scale, q_pos, n_entries, B, Tq, Nmax, m, scores,
                       sbf);
  } else if ((in_t == CSA_BF16 || in_t == CSA_MXFP4) && nI == 64 && cI == 128 &&
             (!pg.paged() || pg.shift >= 4)) {
    // bf16: about two resident blocks per CU over the whole call; a block
    // covers a multiple of 512 entries (MXFP4) or 128 (bf16), whole steps of
    // its 4 waves (bf16 128 entries, MXFP4 256)
    const int step = in_t == CSA_MXFP4 ? 512 : 128;
    // Blocks per CU, measured: bf16 keys about one (each wave streams a long
    // range through its ring; decode_64k 28.7 us against 30.1 at two blocks
    // and 32.2 at four), MXFP4 keys (four waves per SIMD at 128 VGPRs: more
    // VALU work per byte) about two (30.5 us against 30.8 at four, 32.5 at one)
    const int64_t want = in_t == CSA_MXFP4 ? ((int64_t)Nmax * rows + 511) / 512
                                           : ((int64_t)Nmax * rows + 255) / 256;
    int epb = (int)(((want + step - 1) / step) * step);
    epb = epb < 2 * step ? 2 * step : (epb > 8192 ? 8192 : epb);
    dim3 grid((unsigned)(((int64_t)Nmax + epb - 1) / epb * rows));
    const size_t shm = (size_t)epb * (sbf ? 2 : 4);
    if (in_t == CSA_BF16)
      hipLaunchKernelGGL(indexer_mfma_kernel<false>, grid, dim3(IDX_WAVES * 64), shm, s,
                         (const uint8_t*)qI, qI_scale, w, (const uint8_t*)kI, kI_scale, q_pos,
                         n_entries, Tq, Nmax, m, epb, scores, sbf, pg);
    else
      hipLaunchKernelGGL(indexer_mfma_kernel<true>, grid, dim3(IDX_WAVES * 64), shm, s,
                         (const uint8_t*)qI, qI_scale, w, (const uint8_t*)kI, kI_scale, q_pos,
                         n_entries, Tq, Nmax, m, epb, scores, sbf, pg);
  } else {
    dim3 grid((unsigned)(((int64_t)Nmax + 255) / 256 * rows));
    const size_t shm = (size_t)(nI * cI + nI) * sizeof(float);
    hipLaunchKernelGGL(indexer_generic_kernel, grid, dim3(256), shm, s, (const uint8_t*)qI,
                       qI_scale, in_t, w, (const uint8_t*)kI, kI_scale, q_pos, n_entries, Tq, nI,
                       cI, Nmax, m, scores, sbf, pg);
  }
  return hipGetLastError();
}

}  // namespace csa
