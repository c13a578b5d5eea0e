// Projection GEMMs of the splice path: C[m][n] = sum_k A[m][k] * W[n][k]
// (activations times nn.Linear weights, both K-contiguous), fp32 accumulate,
// with the consumer fused into the epilogue:
//   EPI_STORE_F32  C -> fp32 buffer (QKV projection, LM head)
//   EPI_RESID      x += C into the fp32 residual stream (O and down projections)
//   EPI_SWIGLU     silu(C_gate) * C_up -> activation planes (gate/up projection)
//
// bf16 models use the gfx950 matrix cores in bf16
// (v_mfma_f32_16x16x32_bf16).  Weights go from HBM to the matrix cores
// untouched.  Activations arrive as two bf16 planes written by their
// producer, hi = bf16(x) and lo = bf16(x - hi); each weight fragment meets
// both (two products), so the activation operand carries ~17 significant
// bits and the only other rounding is the fp32 accumulation.  The MFMA
// takes the weight fragment as its first operand and the activations as the
// second, so each lane ends up holding four consecutive output columns of
// one row (lane l, register r -> column 4*(l/16)+r, row l%16).
//   * skinny (M <= 16): weight-streaming.  A work-group owns 64 weight
//     rows and a K range; the activation chunk is shared through LDS and
//     each wave streams 16 weight rows into registers (sixteen lanes per
//     row) and transposes them to MFMA fragments through LDS.
//   * tiled (M > 16): a work-group of eight waves owns 256 weight rows and
//     256 (or 128) activation rows; each wave computes all 256 weight rows
//     against its own 32 (or 16) activation rows.  The weight tile is the
//     only operand that goes through LDS (four stages, k steps of 32, or
//     64 for the 128-row tiles, loaded three steps ahead into registers);
//     each wave loads its activation fragments (both planes) straight into
//     registers two steps ahead.  LDS traffic per
//     multiply-add is then set by the weights alone, which keeps the LDS
//     port (128 B/clk/CU) below the matrix-core rate.  When the output has
//     too few tiles to occupy the 256 compute units, K is split over several
//     work-groups per tile; each writes its fp32 partial sums to the
//     workspace and a second kernel adds them in split order and runs the
//     epilogue, so results do not depend on scheduling.  (Handing partials
//     between work-groups inside one kernel would need a device-scope
//     release per work-group, which on this chip writes back the whole L2.)
// fp32 (the small reference-shape path) uses a plain LDS-tiled VALU kernel.
#include "cad_internal.h"

namespace cad {

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Apply the epilogue to four consecutive output columns n .. n+3 of row m.
// For SWIGLU `c` holds the gate values and `cu` the matching up values; the
// activation is written as fp32 or (SPLIT, bf16 models) as bf16 hi / lo planes.
template <int EPI, bool SPLIT>
__device__ __forceinline__ void epi4(const GemmArgs& a, int m, int n, f32x4 c, f32x4 cu) {
  if (m >= a.M) return;
  if (EPI == EPI_ARGMAX && !a.out_f32) return;  // logits not requested
  if (EPI == EPI_STORE_F32 || EPI == EPI_RESID || EPI == EPI_ARGMAX) {
    float* o = a.out_f32 + (int64_t)m * a.ldo + n;
    if (n + 3 < a.N && ((a.ldo & 3) == 0)) {
      f32x4* o4 = (f32x4*)o;
      if (EPI == EPI_RESID) {
        f32x4 v = *o4;
        *o4 = v + c;
      } else {
        *o4 = c;
      }
    } else {
      for (int r = 0; r < 4; ++r)
        if (n + r < a.N) o[r] = (EPI == EPI_RESID) ? o[r] + c[r] : c[r];
    }
  } else if (SPLIT && a.act_f16) {
    // one half plane (the down projection's operand on the tiled path)
    f16_t* o = (f16_t*)a.out_act + (int64_t)m * a.N + n;
    float y[4];
    bool big = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      y[r] = silu_mul(c[r], cu[r]);
      big |= n + r < a.N && !(fabsf(y[r]) <= 65504.f);
    }
    if (big && a.status) atomicOr(a.status, (int32_t)CAD_DEV_F16_RANGE);
    if (n + 3 < a.N && ((a.N & 3) == 0)) {
      const f16x2 h01 = {f2h(y[0]), f2h(y[1])};
      const f16x2 h23 = {f2h(y[2]), f2h(y[3])};
      *(u32x2*)o = u32x2{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)};
    } else {
      for (int r = 0; r < 4; ++r)
        if (n + r < a.N) o[r] = f2h(y[r]);
    }
  } else if (SPLIT) {
    bf16_t* o = (bf16_t*)a.out_act + (int64_t)m * a.N + n;
    bf16_t* ol = (bf16_t*)a.out_act_lo + (int64_t)m * a.N + n;
    if (n + 3 < a.N && ((a.N & 3) == 0)) {
      bf16_t h[4], l[4];
      for (int r = 0; r < 4; ++r) split_bf16(silu_mul(c[r], cu[r]), h[r], l[r]);
      *(u32x2*)o = u32x2{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16)};
      *(u32x2*)ol = u32x2{l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16)};
    } else {
      for (int r = 0; r < 4; ++r)
        if (n + r < a.N) split_bf16(silu_mul(c[r], cu[r]), o[r], ol[r]);
    }
  } else {
    float* o = (float*)a.out_act + (int64_t)m * a.N + n;
    for (int r = 0; r < 4; ++r)
      if (n + r < a.N) o[r] = silu_mul(c[r], cu[r]);
  }
}

// ---- masked-argmax candidates (EPI_ARGMAX, the LM head) ----
// Order: the larger value wins, equal values go to the lower id; id < 0 is
// "no allowed id".  Every scan below visits one lane's columns in increasing
// order with a strict comparison, so within a lane the lowest id of a tie
// is kept, and lanes are merged with the explicit id tie-break.
__device__ __forceinline__ bool cand_better(float v, int i, float bv, int bi) {
  return i >= 0 && (bi < 0 || v > bv || (v == bv && i < bi));
}

// allowed columns among n .. n + 3 of row m (n a multiple of 4, m < M): bit
// r set = column n + r is in the vocabulary and allowed by the mask
__device__ __forceinline__ uint32_t allowed4(const GemmArgs& a, int m, int n) {
  if (n >= a.N) return 0u;
  uint32_t b = a.mask ? (a.mask[(int64_t)m * a.mask_words + (n >> 5)] >> (n & 31)) & 0xFu : 0xFu;
  if (n + 4 > a.N) b &= (1u << (a.N - n)) - 1u;
  return b;
}

// fold four consecutive columns n .. n + 3 (allowed bits `ok`) into (bv, bi)
__device__ __forceinline__ void scan4(f32x4 c, int n, uint32_t ok, float& bv, int& bi) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (((ok >> r) & 1u) && (bi < 0 || c[r] > bv)) {
      bv = c[r];
      bi = n + r;
    }
}

// merge (bv, bi) with the lane `lane ^ off` (a lane swap through LDS hardware)
__device__ __forceinline__ void cand_xor(float& bv, int& bi, int off) {
  const float ov = __shfl_xor(bv, off);
  const int oi = __shfl_xor(bi, off);
  if (cand_better(ov, oi, bv, bi)) {
    bv = ov;
    bi = oi;
  }
}

__device__ __forceinline__ void put_cand(const GemmArgs& a, int c, int m, float bv, int bi) {
  *(u32x2*)(a.cand + 2 * ((int64_t)c * a.M + m)) = u32x2{__float_as_uint(bv), (uint32_t)bi};
}

// ---------------------------------------------------------------------------
// bf16 skinny: M <= 16, weight streaming
// ---------------------------------------------------------------------------
// A work-group of four waves owns 64 weight rows (four 16-row blocks, one
// per wave; for SWIGLU a block is 8 gate rows + the 8 matching up rows) and
// a range of K in chunks of SK_KC.  The activations of a chunk (at most 16
// rows, both planes) are staged once in LDS and shared by the four waves.
// Each wave streams its 16 weight rows (512 B per row and chunk) into
// registers one chunk ahead, sixteen lanes per row per load (256 contiguous
// bytes: HBM streams at ~5 TB/s this way against ~4 TB/s with four lanes
// per row), and turns them into MFMA fragments through a small LDS
// transpose, 256 k at a time.  With K split over S work-groups the partial
// sums go to the workspace and the consumer adds them.
constexpr int SK_WLD = 256 + 8;  // LDS row stride of a half-chunk (256 k) weight transpose (528 B: conflict-free)
// k per chunk.  256 rather than 512: the work-group then needs 150 VGPRs
// and 50 KB of LDS instead of 246 and 66 KB, so three fit per CU instead of
// two, and the weight streams ran faster in every projection (N = 1:
// gate/up 49.6 -> 42.1 us, down 23.7 -> 19.7, QKV 13.9 -> 11.3; step 4.77
// -> 4.31 ms).  The body is written for either width.
constexpr int SK_KC = 256;

// Chunk shapes for KC = 512 or 256 k per chunk.
template <int KC> struct SkShape {
  static constexpr int ALD = KC + 8;              // LDS row stride of the activation chunk (conflict-free)
  static constexpr int PPR = KC / 8;              // 16-byte pieces per activation row and plane
  static constexpr int AIT = 2 * 16 * PPR / 256;  // pieces per thread and chunk, both planes
  static constexpr int NR = AIT / 2;              // activation rows per thread
  static constexpr int RS = 256 / PPR;            // row step between a thread's rows
  static constexpr int NWL = KC / 32;             // 16-byte weight loads per lane and chunk
  static constexpr int NH = KC / 256;             // 256-wide halves per chunk
};

// Staged activation registers of one chunk: the two bf16 planes (AIT
// 16-byte pieces per thread), or (NORM) NR rows of eight fp32 residual
// values (bits) and the eight matching gains; the normalised hi / lo pieces
// of row j then replace its fp32 values in place (x[2j], x[2j + 1]), so the
// stage costs four registers more than the plain one.
template <bool NORM, int KC> struct SkStage { u32x4 r[SkShape<KC>::AIT]; };
template <int KC> struct SkStage<true, KC> { u32x4 x[2 * SkShape<KC>::NR]; u32x4 g; };

template <int EPI, bool NORM, int KC>
__device__ __forceinline__ void gemm_skinny_body(const GemmArgs& a, int n_rg, int splits) {
  using SH = SkShape<KC>;
  __shared__ __attribute__((aligned(16))) bf16_t sa[2][16 * SH::ALD];     // [plane][row][k]
  __shared__ __attribute__((aligned(16))) bf16_t swt[4][16 * SK_WLD];     // per-wave weight transpose
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, i16 = lane & 15;
  const int rg = blockIdx.x % n_rg, sp = blockIdx.x / n_rg;
  const int blk = rg * 4 + wave;  // this wave's 16-row weight block
  const bf16_t* W = (const bf16_t*)a.W;
  // weight row of block row i (clamped: columns past N are computed and dropped)
  auto wrow_of = [&](int i) -> int64_t {
    if (EPI == EPI_SWIGLU) {
      const int col = min(blk * 8 + (i & 7), a.N - 1);
      return (i < 8) ? col : a.up_off + col;
    }
    return min(blk * 16 + i, a.N - 1);
  };
  // load j (0 .. NWL - 1) of a chunk: block row 4 (j % 4) + lane / 16, k
  // offset 128 (j / 4) + 8 (lane % 16) within the chunk
  const bf16_t* wp[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) wp[q] = W + wrow_of(4 * q + g) * a.ldw + 8 * i16;
  const int nch = (a.K + KC - 1) / KC;
  const int c0 = (int)((int64_t)nch * sp / splits), c1 = (int)((int64_t)nch * (sp + 1) / splits);
  // activation staging: piece q = tid + 256*j is 16 bytes: plane q / (16 PPR),
  // row (q / PPR) % 16, k offset 8 * (q % PPR) within the chunk.  Rows >= M
  // and k past K are written as zeros (their products vanish).  With NORM
  // the thread holds the same pieces as fp32 values of rows r0 + RS j
  // (r0 = tid / PPR, j < NR) and writes both planes of each.
  const bf16_t* ap[SH::AIT];
  int aoff[SH::AIT], akk[SH::AIT];
  bool aok[SH::AIT];
#pragma unroll
  for (int j = 0; j < SH::AIT; ++j) {
    const int q = tid + 256 * j;
    const int plane = q / (16 * SH::PPR), row = (q / SH::PPR) % 16, kk = 8 * (q % SH::PPR);
    aoff[j] = plane * (16 * SH::ALD) + row * SH::ALD + kk;
    akk[j] = kk;
    aok[j] = row < a.M;
    ap[j] = (const bf16_t*)(plane ? a.A_lo : a.A) + (int64_t)min(row, a.M - 1) * a.lda + kk;
  }
  const int r0 = tid / SH::PPR, nkk = 8 * (tid % SH::PPR);  // NORM: first row and k offset
  // NORM: 1 / rms of this thread's rows.  Four lanes per row (lane l: row
  // l / 4) load every fourth slice sum (at most 32 slices), all in one round
  // trip, add them in order and then over the four lanes by a fixed
  // butterfly; each thread then fetches its rows' values from those lanes.
  float rsj[SH::NR];
#pragma unroll
  for (int j = 0; j < SH::NR; ++j) rsj[j] = 0.f;
  if constexpr (NORM) {
    const int sub = lane & 3;
    const float* ssr = a.norm_ss + (int64_t)min(lane >> 2, a.M - 1) * a.norm_slices;
    float v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = sub + 4 * t < a.norm_slices ? ssr[sub + 4 * t] : 0.f;
    float tsum = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) tsum += v[t];
    tsum += __shfl_xor(tsum, 1);
    tsum += __shfl_xor(tsum, 2);
    const float rs = 1.0f / sqrtf(tsum / (float)a.K + a.norm_eps);
#pragma unroll
    for (int j = 0; j < SH::NR; ++j) rsj[j] = __shfl(rs, 4 * min(r0 + SH::RS * j, 15));
  }
  auto aload = [&](SkStage<NORM, KC>& st, int c) {
    if constexpr (NORM) {
      const int off = min(c * KC, a.K - 8 - nkk);
      st.g = *(const u32x4*)((const bf16_t*)a.norm_g + off + nkk);
#pragma unroll
      for (int j = 0; j < SH::NR; ++j) {
        const float* xp = (const float*)a.A + (int64_t)min(r0 + SH::RS * j, a.M - 1) * a.lda + off + nkk;
        st.x[2 * j] = *(const u32x4*)xp;
        st.x[2 * j + 1] = *(const u32x4*)(xp + 4);
      }
    } else {
#pragma unroll
      for (int j = 0; j < SH::AIT; ++j) st.r[j] = *(const u32x4*)(ap[j] + min(c * KC, a.K - 8 - akk[j]));
    }
  };
  // NORM: normalise and split the staged fp32 rows, in registers, before the
  // barrier that guards the LDS store: row j's hi piece replaces x[2j] and
  // its lo piece x[2j + 1]; rows >= M skip the work
  auto prep = [&](SkStage<NORM, KC>& st) {
    if constexpr (NORM) {
#pragma unroll
      for (int j = 0; j < SH::NR; ++j) {
        if (r0 + SH::RS * j >= a.M) continue;
        u32x4 hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bf16_t h2[2], l2[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int i = 2 * e + t;
            const float xv = __uint_as_float(st.x[2 * j + i / 4][i % 4]);
            const float gv = __uint_as_float((i & 1) ? (st.g[i / 2] & 0xFFFF0000u) : (st.g[i / 2] << 16));
            split_bf16(xv * rsj[j] * gv, h2[t], l2[t]);
          }
          hi[e] = h2[0] | ((uint32_t)h2[1] << 16);
          lo[e] = l2[0] | ((uint32_t)l2[1] << 16);
        }
        st.x[2 * j] = hi;
        st.x[2 * j + 1] = lo;
      }
    }
  };
  // piece j of the stage: plane j / NR, row r0 + RS (j % NR)
  auto piece = [&](const SkStage<NORM, KC>& st, int j) -> u32x4 {
    if constexpr (NORM) return st.x[j < SH::NR ? 2 * j : 2 * (j - SH::NR) + 1];
    else return st.r[j];
  };
  // unconditional stores (a branch here makes the compiler wait for every
  // load in flight, the next chunk's weights included)
  auto astore = [&](const SkStage<NORM, KC>& st, int c) {
#pragma unroll
    for (int j = 0; j < SH::AIT; ++j) {
      const bool keep = aok[j] && c * KC + akk[j] < a.K;
      *(u32x4*)(&sa[0][0] + aoff[j]) = keep ? piece(st, j) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // weights past K are clamped inside the row; the activations there are zero
  auto wload = [&](u32x4 (&r)[SH::NWL], int c) {
#pragma unroll
    for (int j = 0; j < SH::NWL; ++j)
      r[j] = __builtin_nontemporal_load((const u32x4*)(wp[j & 3] + min(c * KC + 128 * (j >> 2), a.K - 8 - 8 * i16)));
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  bf16_t* tw = &swt[wave][0];
  auto compute = [&](const u32x4 (&w)[SH::NWL]) {
#pragma unroll
    for (int h = 0; h < SH::NH; ++h) {
      // half h: loads 8h .. 8h+7 hold k 256 h .. 256 h + 255 of the chunk
#pragma unroll
      for (int j = 8 * h; j < 8 * h + 8; ++j)
        *(u32x4*)(tw + (4 * (j & 3) + g) * SK_WLD + 128 * ((j >> 2) & 1) + 8 * i16) = w[j];
      const bf16_t* tr = tw + i16 * SK_WLD + 8 * g;
      const bf16_t* sh = &sa[0][0] + i16 * SH::ALD + 256 * h + 8 * g;
      const bf16_t* sl = &sa[1][0] + i16 * SH::ALD + 256 * h + 8 * g;
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) {
        const u32x4 wf = *(const u32x4*)(tr + 32 * s2);
        acc = mfma16_bf(wf, *(const u32x4*)(sh + 32 * s2), acc);
        acc = mfma16_bf(wf, *(const u32x4*)(sl + 32 * s2), acc);
      }
    }
  };
  // Pipeline: the activations of chunk j are loaded two steps ahead and
  // written to LDS between two barriers at the end of step j - 1; the
  // weights of chunk j are loaded at the start of step j - 1.  Activations
  // are issued before weights, so waiting for them never waits for the
  // weights.  Work-groups start their chunk sweep at different chunks
  // (rotated by the row group), spreading the memory channels in use.
  const int ncs = c1 - c0, rot = rg % ncs;
  auto ch = [&](int i) { i = min(i, ncs - 1); return c0 + (i + rot) % ncs; };  // i-th chunk visited
  u32x4 w0[SH::NWL], w1[SH::NWL];
  SkStage<NORM, KC> ra0, ra1;
  // the first weights are requested before the first activations are
  // waited for (loads complete in order, so that wait leaves them in flight)
  aload(ra0, ch(0));
  aload(ra1, ch(1));
  wload(w0, ch(0));
  prep(ra0);
  astore(ra0, ch(0));
  __syncthreads();
  // The loop runs while both of an iteration's weight loads are in range;
  // the last two chunks (or the last one) are finished after it, so no
  // weights are streamed past the last chunk (a clamped repeat would fetch
  // them from HBM again: the loads are non-temporal).
  int i = 0;
  for (; i + 2 < ncs; i += 2) {
    aload(ra0, ch(i + 2));
    wload(w1, ch(i + 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(w0);
    prep(ra1);
    __syncthreads();
    astore(ra1, ch(i + 1));
    __syncthreads();
    aload(ra1, ch(i + 3));
    wload(w0, ch(i + 2));
    __builtin_amdgcn_sched_barrier(0);
    compute(w1);
    prep(ra0);
    __syncthreads();
    astore(ra0, ch(i + 2));
    __syncthreads();
  }
  if (i + 1 < ncs) {
    // chunks i and i + 1 left: w0 holds chunk i, ra1 the activations of i + 1
    wload(w1, ch(i + 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(w0);
    prep(ra1);
    __syncthreads();
    astore(ra1, ch(i + 1));
    __syncthreads();
    compute(w1);
  } else if (i < ncs) {
    compute(w0);
  }
  // lane: activation row m = i16, weight rows 4g + r of the block
  const int m = i16;
  if constexpr (EPI == EPI_ARGMAX) {
    // LM head (never split): logits if requested, then one candidate per
    // row and work-group (its 64 vocabulary ids): the four lane groups of a
    // wave are merged by lane swaps, the four waves through LDS
    const int n = blk * 16 + 4 * g;
    epi4<EPI, true>(a, m, n, acc, acc);
    float bv = 0.f;
    int bi = -1;
    scan4(acc, n, m < a.M ? allowed4(a, m, n) : 0u, bv, bi);
    cand_xor(bv, bi, 16);
    cand_xor(bv, bi, 32);
    __shared__ u32x2 scand[4][16];
    if (g == 0) scand[wave][i16] = u32x2{__float_as_uint(bv), (uint32_t)bi};
    __syncthreads();
    if (tid < 16 && tid < a.M) {
      float cv = __uint_as_float(scand[0][tid][0]);
      int ci = (int)scand[0][tid][1];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const float ov = __uint_as_float(scand[w][tid][0]);
        const int oi = (int)scand[w][tid][1];
        if (cand_better(ov, oi, cv, ci)) { cv = ov; ci = oi; }
      }
      put_cand(a, rg, tid, cv, ci);
    }
  } else if (EPI == EPI_SWIGLU) {
    // lanes g = 0, 1 hold gate rows 4g + r, lanes g + 2 the matching up rows
    f32x4 cu;
#pragma unroll
    for (int r = 0; r < 4; ++r) cu[r] = __shfl_xor(acc[r], 32);
    if (g < 2) epi4<EPI, true>(a, m, blk * 8 + 4 * g, acc, cu);
  } else {
    const int n = blk * 16 + 4 * g;
    if (splits == 1) {
      epi4<EPI, true>(a, m, n, acc, acc);
    } else if (m < a.M && n < a.N) {
      *(f32x4*)(a.split_ws + ((int64_t)sp * a.M + m) * a.N + n) = acc;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 tiled
// ---------------------------------------------------------------------------
constexpr int TK = 32;         // one MFMA k-slice (the split heuristic counts k in these steps)

// Work-group -> (weight tile tn, activation tile tm, k split).  Work-groups
// are dealt to the eight XCDs round-robin (id % 8); each XCD takes a
// contiguous block of the order (split slowest, then weight tile,
// activation tile fastest; the first total % 8 blocks one longer), so the
// work-groups that read one k range of the activations, and those that read
// one weight tile, sit behind the same L2 (with eight splits of 32 tiles,
// one split per XCD: each operand piece comes from HBM once).
__device__ __forceinline__ void gemm_tile_of(int n_tn, int n_tm, int splits, int& tn, int& tm, int& sp) {
  const int id = blockIdx.x;
  const int total = n_tn * n_tm * splits;
  const int x = id % 8;
  const int q = x * (total / 8) + min(x, total % 8) + id / 8;
  tm = q % n_tm;
  tn = (q / n_tm) % n_tn;
  sp = q / (n_tm * n_tn);
}

// F16A: the activations are one half plane (A) instead of two bf16 planes;
// the weight tile is widened from bf16 to half (exact in half's normal
// range) as it is written to LDS and each fragment pair takes one
// v_mfma_f32_16x16x32_f16 product.
// TKK: k per pipeline step.  The 128-row tiles (17-128 rows, weight-bound)
// take 64 (each weight row then arrives as whole 128-byte lines: N = 64 step
// 7.68 -> 7.28 ms); the 256-row tiles keep 32 (registers).
template <int EPI, int TN, int NW, int MB, bool F16A = false, int TKK = (MB == 1 ? 64 : 32)>
__device__ __forceinline__ void gemm_tiled_body(const GemmArgs& a, int n_tn, int n_tm, int splits) {
  constexpr int NT = 64 * NW;       // threads
  constexpr int TM = 16 * MB * NW;  // activation rows per tile (MB 16-row blocks per wave)
  constexpr int NB = TN / 16;       // 16-row weight blocks (every wave covers all of them)
  constexpr int KH = TKK / 32;                  // 32-wide k halves per step
  constexpr int CPR = TKK / 8;                  // 16-byte chunks per weight row and step
  constexpr int WLDK = TKK + 8;                 // LDS row stride of a weight stage (80 or 144 bytes: the 16 rows of a fragment read hit distinct banks)
  constexpr int WCH = (TN * CPR + NT - 1) / NT;  // 16-byte weight chunks per thread per k step
  static_assert(TN % 32 == 0, "whole gate/up block pairs");
  __shared__ __attribute__((aligned(16))) bf16_t sw[4][TN * WLDK];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, i16 = lane & 15;
  int tn, tm, sp;
  gemm_tile_of(n_tn, n_tm, splits, tn, tm, sp);
  const bf16_t* W = (const bf16_t*)a.W;

  // weight staging: chunk c = tid + NT*i is 16 bytes (8 k) of tile row c/4
  const bf16_t* wsrc[WCH];
  int wsoff[WCH];
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    // when the tile's chunks do not divide evenly, the threads past the last
    // chunk load and store the last one again (same data, same place), so
    // every load and store stays unconditional
    const int c = min(tid + NT * i, TN * CPR - 1);
    const int row = c / CPR, col = (c % CPR) * 8;
    wsoff[i] = row * WLDK + col;
    int64_t wr;
    if (EPI == EPI_SWIGLU) {
      // 16-row interleave: even blocks gate, odd blocks up, same output columns
      const int blk = row >> 4, pr = blk >> 1;
      const int j = min(tn * (TN / 2) + pr * 16 + (row & 15), a.N - 1);
      wr = (blk & 1) ? a.up_off + j : j;
    } else {
      wr = min(tn * TN + row, a.N - 1);
    }
    wsrc[i] = W + wr * a.ldw + col;
  }
  // this wave's activation rows wrow0 + 16*mb + i16 (rows past M read row
  // M - 1; their outputs are never stored), k offset 8*g within a step
  const int wrow0 = tm * TM + 16 * MB * wave;
  const bool live = wrow0 < a.M;  // wave-uniform: a wave past M only stages weights
  const bf16_t* ahp[MB];
  const bf16_t* alp[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t off = (int64_t)min(wrow0 + 16 * mb + i16, a.M - 1) * a.lda + 8 * g;
    ahp[mb] = (const bf16_t*)a.A + off;
    alp[mb] = F16A ? ahp[mb] : (const bf16_t*)a.A_lo + off;
  }

  f32x4 acc[NB][MB];
#pragma unroll
  for (int x = 0; x < NB; ++x)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[x][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Every global load is unconditional (indices are clamped instead), so the
  // waits for one stage never cover another stage's loads.
  auto wload = [&](u32x4 (&r)[WCH], int kt) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) r[i] = *(const u32x4*)(wsrc[i] + kt * TKK);
  };
  auto aload = [&](u32x4 (&r)[MB][2 * KH], int kt) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int h = 0; h < KH; ++h) {
        r[mb][2 * h] = *(const u32x4*)(ahp[mb] + kt * TKK + 32 * h);
        if (!F16A) r[mb][2 * h + 1] = *(const u32x4*)(alp[mb] + kt * TKK + 32 * h);
      }
  };
  auto wstore = [&](const u32x4 (&r)[WCH], int buf) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) *(u32x4*)(&sw[buf][wsoff[i]]) = F16A ? bf16x8_to_f16x8(r[i]) : r[i];
  };
  auto compute = [&](int buf, const u32x4 (&ra)[MB][2 * KH]) {
    if (!live) {
      // consume the activation registers anyway: otherwise their loads are
      // still in flight on this path when the next loads reuse the registers,
      // and the compiler guards every later load with a wait for all of them
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int h = 0; h < KH; ++h) {
          if (F16A) asm volatile("" ::"v"(ra[mb][2 * h]));
          else asm volatile("" ::"v"(ra[mb][2 * h]), "v"(ra[mb][2 * h + 1]));
        }
      return;
    }
#pragma unroll
    for (int h = 0; h < KH; ++h)
#pragma unroll
    for (int x = 0; x < NB; ++x) {
      const u32x4 w = *(const u32x4*)(&sw[buf][(x * 16 + i16) * WLDK + 32 * h + g * 8]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if (F16A) {
          acc[x][mb] = mfma16(w, ra[mb][2 * h], acc[x][mb]);
        } else {
          acc[x][mb] = mfma16_bf(w, ra[mb][2 * h], acc[x][mb]);
          acc[x][mb] = mfma16_bf(w, ra[mb][2 * h + 1], acc[x][mb]);
        }
      }
    }
    // issue order: each weight fragment is read from LDS two fragments
    // ahead of the products that use it, so one wave's LDS latency hides
    // behind its own products (left to itself the compiler reads a pair
    // and waits on it at once; gate/up at N = 512 -5 %)
    constexpr int PF = MB * (F16A ? 1 : 2), NF = NB * KH, LA = 2;
    __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);  // LDS reads
#pragma unroll
    for (int i = 0; i < NF - LA; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);  // matrix-core products
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, PF * LA, 0);
  };

  const int nk = a.K / TKK;
  const int kt0 = (int)((int64_t)nk * sp / splits), kt1 = (int)((int64_t)nk * (sp + 1) / splits);
  auto cl = [&](int kt) { return min(kt, kt1 - 1); };  // past the end: load the last step again (never used)
  // Pipeline over four LDS stages and three register buffers per operand:
  // the weights of step j are loaded at the start of step j - 3 into rw[j%3]
  // and written to LDS stage j%4 at the end of step j - 2; the activations
  // of step j are loaded at the start of step j - 2 into ra[j%3].  Stage
  // (r + 2) % 4, written at the end of step r (counted from the split's
  // first step), was last read at step r - 2, so one barrier after every
  // odd step keeps both orders: every wave has left step r - 2 before any
  // wave writes at the end of step r, and a stage written at the end of
  // step r is read at step r + 2 after a barrier (half the barriers of
  // three stages: gate/up at N = 512 -2 %).  The prologue issues its loads
  // in the order the loop does, so the loop is entered with the same loads
  // in flight as it is re-entered.
  u32x4 rw0[WCH], rw1[WCH], rw2[WCH], ra0[MB][2 * KH], ra1[MB][2 * KH], ra2[MB][2 * KH];
  wload(rw0, kt0);
  wload(rw1, cl(kt0 + 1));
  aload(ra0, kt0);
  wload(rw2, cl(kt0 + 2));
  aload(ra1, cl(kt0 + 1));
  wstore(rw0, 0);
  wstore(rw1, 1);
  __syncthreads();
#define CAD_GEMM_STEP(KT, RW_NEW, RA_NEW, RA_CUR, RW_OUT)     \
  wload(RW_NEW, cl((KT) + 3));                                  \
  aload(RA_NEW, cl((KT) + 2));                                  \
  __builtin_amdgcn_sched_barrier(0);                            \
  compute(((KT) - kt0) & 3, RA_CUR);                            \
  __builtin_amdgcn_sched_barrier(0);                            \
  wstore(RW_OUT, ((KT) - kt0 + 2) & 3);                         \
  if (((KT) - kt0) & 1) __syncthreads();
  // three steps per iteration, no exit in between (every path back to the
  // loop head has the same loads in flight); up to two more steps after it
  int kt = kt0;
  for (; kt + 2 < kt1; kt += 3) {
    CAD_GEMM_STEP(kt, rw0, ra2, ra0, rw2)
    CAD_GEMM_STEP(kt + 1, rw1, ra0, ra1, rw0)
    CAD_GEMM_STEP(kt + 2, rw2, ra1, ra2, rw1)
  }
  if (kt < kt1) {
    CAD_GEMM_STEP(kt, rw0, ra2, ra0, rw2)
  }
  if (kt + 1 < kt1) {
    CAD_GEMM_STEP(kt + 1, rw1, ra0, ra1, rw0)
  }
#undef CAD_GEMM_STEP
  // epilogue: acc[x][mb] lane -> weight rows 16x + 4g + r, activation row wrow0 + 16mb + i16
  auto emit = [&](int x, int mb, f32x4 c, f32x4 cu) {
    const int m = wrow0 + 16 * mb + i16;
    if (EPI == EPI_SWIGLU)
      epi4<EPI, true>(a, m, tn * (TN / 2) + (x >> 1) * 16 + 4 * g, c, cu);  // block x: gate, x + 1: up
    else
      epi4<EPI, true>(a, m, tn * TN + x * 16 + 4 * g, c, c);
  };
  constexpr int XS = (EPI == EPI_SWIGLU) ? 2 : 1;
  if (!live) return;
  if (splits > 1) {
    // partial sums of this k split -> workspace [split][M][ncols] (fp32; for
    // SWIGLU gate columns 0..N-1 and up columns N..2N-1); a separate kernel
    // adds the splits in order and runs the epilogue
    const int ncols = (EPI == EPI_SWIGLU) ? 2 * a.N : a.N;
    float* ws = a.split_ws + (int64_t)sp * a.M * ncols;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = wrow0 + 16 * mb + i16;
      if (m >= a.M) continue;
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        // output column of this fragment (N is a multiple of 64 on this
        // path, so a group of four never straddles it)
        const int j = (EPI == EPI_SWIGLU) ? tn * (TN / 2) + (x >> 1) * 16 + 4 * g : tn * TN + x * 16 + 4 * g;
        if (j >= a.N) continue;
        const int n = (EPI == EPI_SWIGLU && (x & 1)) ? a.N + j : j;
        *(f32x4*)(ws + (int64_t)m * ncols + n) = acc[x][mb];
      }
    }
    return;
  }
  if constexpr (EPI == EPI_ARGMAX) {
    // LM head: logits if requested, then one candidate per row and weight
    // tile (TN vocabulary ids); a lane scans its 16 fragments in increasing
    // column order, the four lane groups of a row are merged by lane swaps
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = wrow0 + 16 * mb + i16;
      const int mc = min(m, a.M - 1);
      float bv = 0.f;
      int bi = -1;
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        const int n = tn * TN + x * 16 + 4 * g;
        epi4<EPI, true>(a, m, n, acc[x][mb], acc[x][mb]);
        scan4(acc[x][mb], n, allowed4(a, mc, n), bv, bi);
      }
      cand_xor(bv, bi, 16);
      cand_xor(bv, bi, 32);
      if (g == 0 && m < a.M) put_cand(a, tn, m, bv, bi);
    }
    return;
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int x = 0; x < NB; x += XS) emit(x, mb, acc[x][mb], acc[x + XS - 1][mb]);
}

// ---------------------------------------------------------------------------
// fp32 VALU path: 64x64 tile, 256 threads, 4x4 outputs each
// ---------------------------------------------------------------------------
template <int EPI>
__device__ __forceinline__ void gemm_f32_body(const GemmArgs& a) {
  __shared__ float sa[16][64 + 1];
  __shared__ float sw[16][64 + 1];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;  // 16 x 16 threads
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const float* A = (const float*)a.A;
  const float* W = (const float*)a.W;
  float acc[4][4] = {};
  float accu[4][4] = {};
  for (int k0 = 0; k0 < a.K; k0 += 16) {
    // load A tile [64 rows][16 k] and W tile [64 cols][16 k] (both transposed into LDS)
    for (int i = tid; i < 64 * 16; i += 256) {
      const int r = i / 16, kk = i % 16;
      const int m = m0 + r, k = k0 + kk;
      sa[kk][r] = (m < a.M && k < a.K) ? A[(int64_t)m * a.lda + k] : 0.f;
      const int n = min(n0 + r, a.N - 1);
      sw[kk][r] = (k < a.K) ? W[(int64_t)n * a.ldw + k] : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], wv[4];
      for (int i = 0; i < 4; ++i) { av[i] = sa[kk][ty * 4 + i]; wv[i] = sw[kk][tx * 4 + i]; }
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] += av[i] * wv[j];
    }
    __syncthreads();
    if (EPI == EPI_SWIGLU) {
      for (int i = tid; i < 64 * 16; i += 256) {
        const int r = i / 16, kk = i % 16;
        const int k = k0 + kk;
        const int n = min(n0 + r, a.N - 1);
        sw[kk][r] = (k < a.K) ? W[(a.up_off + n) * a.ldw + k] : 0.f;
      }
      __syncthreads();
      for (int kk = 0; kk < 16; ++kk) {
        float av[4], wv[4];
        for (int i = 0; i < 4; ++i) { av[i] = sa[kk][ty * 4 + i]; wv[i] = sw[kk][tx * 4 + i]; }
        for (int i = 0; i < 4; ++i)
          for (int j = 0; j < 4; ++j) accu[i][j] += av[i] * wv[j];
      }
      __syncthreads();
    }
  }
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    f32x4 c = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
    f32x4 cu = {accu[i][0], accu[i][1], accu[i][2], accu[i][3]};
    epi4<EPI, false>(a, m, n0 + tx * 4, c, cu);
    if constexpr (EPI == EPI_ARGMAX) {
      // one candidate per row and 64-column tile: the 16 threads of a row
      // (consecutive lanes tx = 0..15) merged by lane swaps
      float bv = 0.f;
      int bi = -1;
      scan4(c, n0 + tx * 4, m < a.M ? allowed4(a, m, n0 + tx * 4) : 0u, bv, bi);
      for (int off = 1; off < 16; off <<= 1) cand_xor(bv, bi, off);
      if (tx == 0 && m < a.M) put_cand(a, blockIdx.x, m, bv, bi);
    }
  }
}

// One named kernel per projection and path, so that profiles attribute time
// to the projection (qkv, o, gate_up, down, lm_head) rather than to a shared
// template instance.
// Sum of the k-split partials in split order, then the epilogue; one
// thread per four consecutive output columns of one row.
template <int EPI>
__device__ __forceinline__ void gemm_reduce_body(const GemmArgs& a, int splits) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // group of four columns
  const int groups = a.N / 4;
  if (q >= (int64_t)a.M * groups) return;
  const int m = (int)(q / groups), n = (int)(q % groups) * 4;
  const int ncols = (EPI == EPI_SWIGLU) ? 2 * a.N : a.N;
  const int64_t plane = (int64_t)a.M * ncols;
  const float* p = a.split_ws + (int64_t)m * ncols + n;
  f32x4 c = *(const f32x4*)p, cu = c;
  if (EPI == EPI_SWIGLU) cu = *(const f32x4*)(p + a.N);
  for (int s = 1; s < splits; ++s) {
    c += *(const f32x4*)(p + s * plane);
    if (EPI == EPI_SWIGLU) cu += *(const f32x4*)(p + s * plane + a.N);
  }
  epi4<EPI, true>(a, m, n, c, cu);
}

// The LM head after a k split: one work-group of 256 threads per (row m =
// blockIdx.y, 1024-column chunk blockIdx.x); each thread adds the partials
// of four consecutive columns in split order, stores the logits if
// requested and scans them; the chunk's candidate is merged over the
// work-group (lane swaps, then the four waves in order through LDS).
constexpr int REDUCE_ARGMAX_COLS = 1024;
__device__ __forceinline__ void gemm_reduce_argmax_body(const GemmArgs& a, int splits) {
  const int m = blockIdx.y, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n = blockIdx.x * REDUCE_ARGMAX_COLS + 4 * t;
  float bv = 0.f;
  int bi = -1;
  if (n < a.N) {
    const int64_t plane = (int64_t)a.M * a.N;
    const float* p = a.split_ws + (int64_t)m * a.N + n;
    f32x4 c = *(const f32x4*)p;
    for (int sp = 1; sp < splits; ++sp) c += *(const f32x4*)(p + sp * plane);
    epi4<EPI_ARGMAX, true>(a, m, n, c, c);
    scan4(c, n, allowed4(a, m, n), bv, bi);
  }
  for (int off = 1; off < 64; off <<= 1) cand_xor(bv, bi, off);
  __shared__ u32x2 sc[4];
  if (lane == 0) sc[wave] = u32x2{__float_as_uint(bv), (uint32_t)bi};
  __syncthreads();
  if (t == 0) {
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float ov = __uint_as_float(sc[w][0]);
      const int oi = (int)sc[w][1];
      if (cand_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    put_cand(a, blockIdx.x, m, bv, bi);
  }
}

__global__ void __launch_bounds__(256) k_gemm_reduce_argmax_lm_head(GemmArgs a, int splits) {
  gemm_reduce_argmax_body(a, splits);
}

// Tiled shapes: eight waves (two per SIMD) of 32 activation rows each (256
// per tile), and for spans of 17-128 rows eight waves of 16 rows (128 per
// tile; four waves of 32 rows left one wave per SIMD with nothing to hide
// its latency).  Weight rows per tile: 256, except gate/up with 224 (112
// gate + 112 up columns: 14336 columns make 128 tiles, so two row tiles
// fill the 256 CUs exactly where 256-row tiles left 32 idle) and QKV with
// 192 (6144 rows: 32 tiles; four k splits of two row tiles fill the CUs,
// where 256-row tiles with five splits left 16 idle).
constexpr int TILE_N = 256;
constexpr int TN8_GATE_UP = 224, TN8_QKV = 192;
#define CAD_GEMM_KERNELS(NAME, EPI, TN8)                                                   \
  __global__ void __launch_bounds__(512) k_gemm_##NAME(GemmArgs a, int n_tn, int n_tm, int splits) { \
    gemm_tiled_body<EPI, TN8, 8, 2>(a, n_tn, n_tm, splits);                                \
  }                                                                                        \
  __global__ void __launch_bounds__(512) k_gemm_s_##NAME(GemmArgs a, int n_tn, int n_tm, int splits) { \
    gemm_tiled_body<EPI, TN8, 8, 1>(a, n_tn, n_tm, splits);                                \
  }                                                                                        \
  __global__ void __launch_bounds__(256) k_gemm_reduce_##NAME(GemmArgs a, int splits) {    \
    gemm_reduce_body<EPI>(a, splits);                                                      \
  }                                                                                        \
  __global__ void __launch_bounds__(256, 2) k_gemv_##NAME(GemmArgs a, int n_rg, int splits) { \
    gemm_skinny_body<EPI, false, SK_KC>(a, n_rg, splits);                                  \
  }                                                                                        \
  __global__ void __launch_bounds__(256, 2) k_gemvn_##NAME(GemmArgs a, int n_rg, int splits) { \
    gemm_skinny_body<EPI, true, SK_KC>(a, n_rg, splits);                                   \
  }                                                                                        \
  __global__ void __launch_bounds__(256) k_gemm_f32_##NAME(GemmArgs a) { gemm_f32_body<EPI>(a); }

CAD_GEMM_KERNELS(qkv, EPI_STORE_F32, TN8_QKV)
CAD_GEMM_KERNELS(o, EPI_RESID, TILE_N)
CAD_GEMM_KERNELS(gate_up, EPI_SWIGLU, TN8_GATE_UP)
CAD_GEMM_KERNELS(down, EPI_RESID, TILE_N)
CAD_GEMM_KERNELS(lm_head, EPI_ARGMAX, TILE_N)
#undef CAD_GEMM_KERNELS
// the O projection on 128-row weight tiles (where use_n128 picks them): at
// 17-128 rows its 4096 columns then make 32 tiles and eight k splits fill
// the 256 CUs (256-row tiles left half of them idle at that many rows)
__global__ void __launch_bounds__(512) k_gemm_s_o_n128(GemmArgs a, int n_tn, int n_tm, int splits) {
  gemm_tiled_body<EPI_RESID, 128, 8, 1>(a, n_tn, n_tm, splits);
}
// QKV at 17-128 rows on 128-row weight tiles: 48 tiles of five k splits
// instead of 32 of eight, so the rotary kernel adds five partial planes
// instead of eight (N = 128: rotary 12.4 -> 11.0 us, QKV unchanged)
__global__ void __launch_bounds__(512) k_gemm_s_qkv_n128(GemmArgs a, int n_tn, int n_tm, int splits) {
  gemm_tiled_body<EPI_STORE_F32, 128, 8, 1>(a, n_tn, n_tm, splits);
}
// gate/up on 128-row weight tiles (64 SwiGLU columns; where fuller_n128
// picks them)
__global__ void __launch_bounds__(512) k_gemm_s_gate_up_n128(GemmArgs a, int n_tn, int n_tm, int splits) {
  gemm_tiled_body<EPI_SWIGLU, 128, 8, 1>(a, n_tn, n_tm, splits);
}
// the down projection over a single half activation plane (act_f16)
__global__ void __launch_bounds__(512) k_gemm_down_h(GemmArgs a, int n_tn, int n_tm, int splits) {
  gemm_tiled_body<EPI_RESID, TILE_N, 8, 2, true>(a, n_tn, n_tm, splits);
}
__global__ void __launch_bounds__(512) k_gemm_s_down_h(GemmArgs a, int n_tn, int n_tm, int splits) {
  gemm_tiled_body<EPI_RESID, TILE_N, 8, 1, true>(a, n_tn, n_tm, splits);
}
// the same at 17-128 rows on 128-row weight tiles: 32 tiles of eight k
// splits instead of 16 of sixteen, so half the partial planes for the norm
// that adds them (N = 128: step 8.81 -> 8.59 ms; N = 64: 6.94 -> 6.77 ms)
__global__ void __launch_bounds__(512) k_gemm_s_down_h_n128(GemmArgs a, int n_tn, int n_tm, int splits) {
  gemm_tiled_body<EPI_RESID, 128, 8, 1, true>(a, n_tn, n_tm, splits);
}

// Tiles and k splits of a tiled launch: one work-group per CU at a time,
// so K is split while the split tiles still fit the 256 compute units at
// once, keeping the partials within the workspace and at least 16 k steps
// of 32 per split, or 8 at up to 128 rows (whose partial planes are small:
// the 1B shape at N = 64 1.71 -> 1.69 ms, the 7B tensor-parallel share at
// N = 128 4.09 -> 3.93 ms; at N = 256 the 1B shape ran 7 % slower with 8).
struct TiledPlan {
  int n_tn, n_tm, splits;
  int wgs() const { return n_tn * n_tm * splits; }
};
static TiledPlan tiled_plan(const GemmArgs& a, int cols_per_tile, int tm_rows, bool swiglu) {
  TiledPlan p;
  p.n_tn = (a.N + cols_per_tile - 1) / cols_per_tile;
  p.n_tm = (a.M + tm_rows - 1) / tm_rows;
  p.splits = 1;
  const int tiles = p.n_tn * p.n_tm, nk = a.K / TK, min_steps = a.M <= 128 ? 8 : 16;
  const int64_t split_floats = (int64_t)a.M * a.N * (swiglu ? 2 : 1);
  if (a.split_ws && a.N % 64 == 0)
    while (tiles * (p.splits + 1) <= 256 && nk / (p.splits + 1) >= min_steps &&
           split_floats * (p.splits + 1) <= a.split_cap)
      ++p.splits;
  return p;
}

// QKV, O and down (bf16, more than 16 rows) on 128 x 128 tiles (128 weight
// rows, 128 activation rows): always at 17-128 rows (fewer k splits, so
// fewer partial planes for the consumer; measured faster), and above that
// wherever the default tiles leave more compute units idle (the 1B shape at
// N = 256: its 2048-wide K allows at most four splits, so QKV and O made 64
// work-groups and down 128).
// Whether the 128 x 128 tiles make more work-groups than the default tiles
// (both counted up to the 256 that run at once).  Gate/up takes them only
// then (the 1B shape at N = 256: 222 work-groups with three k splits and a
// reduce kernel, against 256 tiles with neither: 2.72 -> 2.51 ms; at 17-128
// rows of the 7B shape they measured slower).
static bool fuller_n128(const GemmArgs& a, int default_cols, bool default_rows128, bool swiglu) {
  const int c = swiglu ? 64 : 128;
  return min(tiled_plan(a, c, 128, swiglu).wgs(), 256) >
         min(tiled_plan(a, default_cols, (a.M <= 128 || default_rows128) ? 128 : 256, swiglu).wgs(), 256);
}
static bool use_n128(const GemmArgs& a, int default_cols, bool default_rows128) {
  if (a.M <= 16) return false;
  if (a.M <= 128) return true;
  return fuller_n128(a, default_cols, default_rows128, false);
}

typedef void (*TiledFn)(GemmArgs, int, int, int);
typedef void (*ReduceFn)(GemmArgs, int);
typedef void (*SkinnyFn)(GemmArgs, int, int);
typedef void (*PlainFn)(GemmArgs);

// partials != nullptr (store / residual epilogues only): a k-split result
// may be left as *partials fp32 planes [split][M][N] in a.split_ws for the
// consumer to add (in split order); *partials = 0 when the epilogue ran.
template <int EPI>
static hipError_t launch_epi(int dtype, const GemmArgs& a, TiledFn tiled8, int tn8, TiledFn tiled_s, ReduceFn reduce,
                             SkinnyFn skinny, SkinnyFn skinny_norm, PlainFn f32, int* partials, hipStream_t s,
                             bool rows128 = false) {
  if (partials) *partials = 0;
  if (a.norm_ss && (dtype != CAD_BF16 || a.M > 16 || a.norm_slices > 32)) return hipErrorInvalidValue;
  if (EPI == EPI_ARGMAX && (!a.cand || !a.n_cand || (a.mask && a.mask_words * 32 < a.N)))
    return hipErrorInvalidValue;
  const bool leave = partials != nullptr && EPI != EPI_SWIGLU && a.split_ws != nullptr && a.N % 4 == 0;
  if (dtype == CAD_F32) {
    dim3 grid((a.N + 63) / 64, (a.M + 63) / 64);
    hipLaunchKernelGGL(f32, grid, dim3(256), 0, s, a);
    if (EPI == EPI_ARGMAX) *a.n_cand = (int)grid.x;
  } else if (a.M <= 16) {
    const int nblk = (EPI == EPI_SWIGLU) ? (a.N + 7) / 8 : (a.N + 15) / 16;
    const int n_rg = (nblk + 3) / 4;
    const int nch = (a.K + SK_KC - 1) / SK_KC;
    // when the consumer adds partial sums: the most splits (whole chunks,
    // within the partial workspace) -- work-groups that stream little each
    // keep the most loads in flight for the weights (measured: down at N = 1,
    // 28 x 64 work-groups of 512 k ran at 5 TB/s, 8 x 64 of 1536-2048 k at
    // 4.2) -- but at most one split per 512 k: a split work-group then
    // streams two 256-wide chunks, and the consumer adds no more partial
    // planes than one per 512 k (one per 256 k made RoPE's staging 3 us
    // slower)
    int splits = 1;
    const int max_splits = (a.K + 511) / 512;
    if (leave)
      for (int c = min(nch, max_splits); c > 1; --c)
        if (nch % c == 0 && (int64_t)c * a.M * a.N <= a.split_cap) {
          splits = c;
          break;
        }
    hipLaunchKernelGGL(a.norm_ss ? skinny_norm : skinny, dim3(n_rg * splits), dim3(256), 0, s, a, n_rg, splits);
    if (splits > 1) *partials = splits;
    if (EPI == EPI_ARGMAX) *a.n_cand = n_rg;  // one candidate per 64 vocabulary ids (never split)
  } else {
    // rows128: 128-row activation tiles at any row count (the O projection:
    // as fast as 256-row tiles at N = 512, and half the k splits, so half
    // the partial planes for the RMSNorm that adds them: 15.1 -> 12.9 us)
    const bool small = a.M <= 128 || rows128;
    const int tm_rows = small ? 128 : 256;
    const TiledPlan pl = tiled_plan(a, (EPI == EPI_SWIGLU) ? tn8 / 2 : tn8, tm_rows, EPI == EPI_SWIGLU);
    const int n_tn = pl.n_tn, n_tm = pl.n_tm, tiles = n_tn * n_tm, splits = pl.splits;
    hipLaunchKernelGGL(small ? tiled_s : tiled8, dim3(tiles * splits), dim3(512), 0, s, a, n_tn, n_tm,
                       splits);
    if (EPI == EPI_ARGMAX) *a.n_cand = n_tn;  // one candidate per weight tile
    if (splits > 1) {
      if (leave) {
        *partials = splits;
      } else if (EPI == EPI_ARGMAX) {
        const dim3 grid((unsigned)((a.N + REDUCE_ARGMAX_COLS - 1) / REDUCE_ARGMAX_COLS), (unsigned)a.M);
        hipLaunchKernelGGL(k_gemm_reduce_argmax_lm_head, grid, dim3(256), 0, s, a, splits);
        *a.n_cand = (int)grid.x;
      } else {
        const int64_t groups = (int64_t)a.M * (a.N / 4);
        hipLaunchKernelGGL(reduce, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s, a, splits);
      }
    }
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, int role, const GemmArgs& a, hipStream_t s, int* partials) {
  switch (role) {
#define CAD_LAUNCH(EPI, NAME, TN8) \
  launch_epi<EPI>(dtype, a, k_gemm_##NAME, TN8, k_gemm_s_##NAME, k_gemm_reduce_##NAME, k_gemv_##NAME, k_gemvn_##NAME, \
                  k_gemm_f32_##NAME, partials, s)
    case GEMM_QKV:
      if (dtype == CAD_BF16 && use_n128(a, TN8_QKV, false))
        return launch_epi<EPI_STORE_F32>(dtype, a, k_gemm_qkv, 128, k_gemm_s_qkv_n128, k_gemm_reduce_qkv, k_gemv_qkv,
                                         k_gemvn_qkv, k_gemm_f32_qkv, partials, s, true);
      return CAD_LAUNCH(EPI_STORE_F32, qkv, TN8_QKV);
    case GEMM_O:
      if (dtype == CAD_BF16 && use_n128(a, TILE_N, true))
        return launch_epi<EPI_RESID>(dtype, a, k_gemm_o, 128, k_gemm_s_o_n128, k_gemm_reduce_o, k_gemv_o,
                                     k_gemvn_o, k_gemm_f32_o, partials, s, true);
      return launch_epi<EPI_RESID>(dtype, a, k_gemm_o, TILE_N, k_gemm_s_o, k_gemm_reduce_o, k_gemv_o, k_gemvn_o,
                                   k_gemm_f32_o, partials, s, true);
    case GEMM_GATE_UP:
      if (dtype == CAD_BF16 && a.M > 16 && fuller_n128(a, TN8_GATE_UP / 2, false, true))
        return launch_epi<EPI_SWIGLU>(dtype, a, k_gemm_gate_up, 128, k_gemm_s_gate_up_n128, k_gemm_reduce_gate_up,
                                      k_gemv_gate_up, k_gemvn_gate_up, k_gemm_f32_gate_up, partials, s, true);
      return CAD_LAUNCH(EPI_SWIGLU, gate_up, TN8_GATE_UP);
    case GEMM_DOWN:
      if (a.act_f16) {
        if (dtype != CAD_BF16 || a.M <= 16) return hipErrorInvalidValue;
        if (use_n128(a, TILE_N, false))
          return launch_epi<EPI_RESID>(dtype, a, k_gemm_down_h, 128, k_gemm_s_down_h_n128, k_gemm_reduce_down,
                                       k_gemv_down, k_gemvn_down, k_gemm_f32_down, partials, s, true);
        return launch_epi<EPI_RESID>(dtype, a, k_gemm_down_h, TILE_N, k_gemm_s_down_h, k_gemm_reduce_down,
                                     k_gemv_down, k_gemvn_down, k_gemm_f32_down, partials, s);
      }
      return CAD_LAUNCH(EPI_RESID, down, TILE_N);
    default: return CAD_LAUNCH(EPI_ARGMAX, lm_head, TILE_N);
#undef CAD_LAUNCH
  }
}

}  // namespace cad
