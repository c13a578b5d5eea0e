// Projection GEMMs of the splice path: C[m][n] = sum_k A[m][k] * W[n][k]
// (activations times nn.Linear weights, both K-contiguous), fp32 accumulate,
// with the consumer fused into the epilogue:
//   EPI_STORE_F32  C -> fp32 buffer (QKV projection, LM head)
//   EPI_RESID      x += C into the fp32 residual stream (O and down projections)
//   EPI_SWIGLU     silu(C_gate) * C_up -> fp32 activation (gate/up projection)
//
// bf16 models use the gfx950 matrix cores in half precision
// (v_mfma_f32_16x16x32_f16).  Weights stay bf16 in HBM and are widened to
// half (exact in half's normal range).  Activations arrive as two half
// planes written by their producer: the "hi" part and the half-rounded
// remainder "lo"; each weight fragment meets both (two matrix-core
// products), so the activation operand carries ~22 significant bits and the
// only rounding left is the fp32 accumulation.  The MFMA takes the weight tile as its first operand and
// the activations as the second, so each lane ends up holding four
// consecutive output columns of one row (lane l, register r -> column
// 4*(l/16)+r, row l%16).
//   * skinny (M <= 16): weight-streaming.  A work-group owns 16 output
//     columns (32 weight rows for SWIGLU); its four waves split K and are
//     reduced through LDS in a fixed order.  Every lane loads 32 contiguous
//     bytes of a weight row per 64-wide k step straight into registers.
//   * tiled (M > 16): 128x128 output tile per 256-thread work-group, K in
//     steps of 32 staged through double-buffered LDS (weights, activation hi,
//     activation lo planes).  When the output has too few tiles to occupy the 256
//     compute units, K is split over up to eight work-groups per tile; each
//     writes its fp32 partial tile to the workspace and the last to arrive
//     (per-tile counter) sums the partials in split order and runs the
//     epilogue, so results do not depend on scheduling.  The global loads run
//     two k steps ahead of the matrix cores (two register stages in front of
//     the LDS double buffer).
// fp32 (the small reference-shape path) uses a plain LDS-tiled VALU kernel.
#include "cad_internal.h"

namespace cad {

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }



// Apply the epilogue to four consecutive output columns n .. n+3 of row m.
// For SWIGLU `c` holds the gate values and `cu` the matching up values; the
// activation is written as fp32 or (SPLIT, bf16 models) as half hi / lo planes.
template <int EPI, bool SPLIT>
__device__ __forceinline__ void epi4(const GemmArgs& a, int m, int n, f32x4 c, f32x4 cu) {
  if (m >= a.M) return;
  if (EPI == EPI_STORE_F32 || EPI == EPI_RESID) {
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
  } else if (SPLIT) {
    f16_t* o = (f16_t*)a.out_act + (int64_t)m * a.N + n;
    f16_t* ol = (f16_t*)a.out_act_lo + (int64_t)m * a.N + n;
    for (int r = 0; r < 4; ++r)
      if (n + r < a.N) split_f16(silu_mul(c[r], cu[r]), o[r], ol[r]);
  } else {
    float* o = (float*)a.out_act + (int64_t)m * a.N + n;
    for (int r = 0; r < 4; ++r)
      if (n + r < a.N) o[r] = silu_mul(c[r], cu[r]);
  }
}

// ---------------------------------------------------------------------------
// bf16 skinny: M <= 16
// ---------------------------------------------------------------------------
constexpr int SK_WAVES = 4;

template <int EPI>
__device__ __forceinline__ void gemm_skinny_body(const GemmArgs& a) {
  constexpr int NB = (EPI == EPI_SWIGLU) ? 2 : 1;  // 16-row weight blocks per work-group
  __shared__ f32x4 part[SK_WAVES][NB][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, i16 = lane & 15;
  const int n0 = blockIdx.x * 16;
  const bf16_t* W = (const bf16_t*)a.W;
  // this lane's weight rows (clamped: columns past N are computed and dropped)
  const int ncol = min(n0 + i16, a.N - 1);
  const bf16_t* wrow[NB];
  wrow[0] = W + (int64_t)ncol * a.ldw;
  if (NB == 2) wrow[NB - 1] = W + (a.up_off + ncol) * a.ldw;
  // activation rows past M read row M - 1 and are dropped by the epilogue
  const int64_t aoff = (int64_t)min(i16, a.M - 1) * a.lda;
  const f16_t* arow_hi = (const f16_t*)a.A + aoff;
  const f16_t* arow_lo = (const f16_t*)a.A_lo + aoff;
  // k split across waves in units of 64
  const int kp_total = a.K / 64;
  const int kp0 = (kp_total * wave) / SK_WAVES, kp1 = (kp_total * (wave + 1)) / SK_WAVES;
  f32x4 acc[NB];
  for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // 16 activations at k .. k + 15: (hi, lo) operands of the two products
  auto act16 = [&](int k, u32x4 (&hi)[2], u32x4 (&lo)[2]) {
    const u32x4* qh = (const u32x4*)(arow_hi + k);
    const u32x4* ql = (const u32x4*)(arow_lo + k);
    hi[0] = qh[0];
    hi[1] = qh[1];
    lo[0] = ql[0];
    lo[1] = ql[1];
  };
  constexpr int U = 4;
  int kp = kp0;
  for (; kp + U <= kp1; kp += U) {
    u32x4 wv[NB][U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (kp + u) * 64 + g * 16;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const u32x4* p = (const u32x4*)(wrow[b] + k);
        wv[b][u][0] = __builtin_nontemporal_load(p);
        wv[b][u][1] = __builtin_nontemporal_load(p + 1);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      u32x4 ah[2], al[2];
      act16((kp + u) * 64 + g * 16, ah, al);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 w = bf16x8_to_f16x8(wv[b][u][h]);
          acc[b] = mfma16(w, ah[h], acc[b]);
          acc[b] = mfma16(w, al[h], acc[b]);
        }
    }
  }
  for (; kp < kp1; ++kp) {
    const int k = kp * 64 + g * 16;
    u32x4 ah[2], al[2];
    act16(k, ah, al);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const u32x4* p = (const u32x4*)(wrow[b] + k);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 w = bf16x8_to_f16x8(p[h]);
        acc[b] = mfma16(w, ah[h], acc[b]);
        acc[b] = mfma16(w, al[h], acc[b]);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) part[wave][b][lane] = acc[b];
  __syncthreads();
  if (wave == 0) {
    f32x4 s[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      s[b] = part[0][b][lane];
      for (int w = 1; w < SK_WAVES; ++w) s[b] += part[w][b][lane];
    }
    // lane holds C^T rows n0 + 4g + r (output columns) of activation row i16
    epi4<EPI, true>(a, i16, n0 + 4 * g, s[0], s[NB - 1]);
  }
}

// ---------------------------------------------------------------------------
// bf16 tiled: 128 (weight rows) x 128 (activation rows) per work-group
// ---------------------------------------------------------------------------
constexpr int TB = 128, TK = 32, TLD = TK + 8;  // 80-byte rows: 16-row fragment reads hit distinct banks

// Work-group -> (weight tile tn, activation tile tm, k split), weight tile
// fastest: the work-groups resident at one time share a few activation
// tiles, and each XCD (work-groups are dealt to the eight XCDs round-robin)
// sees every eighth weight tile for all of them.
__device__ __forceinline__ void gemm_tile_of(int n_tn, int n_tm, int& tn, int& tm, int& sp) {
  const int id = blockIdx.x;
  tn = id % n_tn;
  tm = (id / n_tn) % n_tm;
  sp = id / (n_tn * n_tm);
}

template <int EPI>
__device__ __forceinline__ void gemm_tiled_body(const GemmArgs& a, int n_tn, int n_tm, int splits) {
  __shared__ __attribute__((aligned(16))) f16_t sw[2][TB * TLD];
  __shared__ __attribute__((aligned(16))) f16_t sah[2][TB * TLD];
  __shared__ __attribute__((aligned(16))) f16_t sal[2][TB * TLD];
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, i16 = lane & 15;
  const int wn = (wave & 1) * 64;   // wave's offset in the weight-row dim of the tile
  const int wm = (wave >> 1) * 64;  // wave's offset in the activation-row dim
  int tn, tm, sp;
  gemm_tile_of(n_tn, n_tm, tn, tm, sp);
  const bf16_t* W = (const bf16_t*)a.W;

  // global -> LDS assignment per 32-wide k step: weights 2 chunks of 8 bf16
  // per thread (4 threads per row), activations likewise per plane
  const bf16_t* wsrc[2];
  int wsoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i;
    const int row = c >> 2, col = (c & 3) * 8;
    wsoff[i] = row * TLD + col;
    int64_t wr;
    if (EPI == EPI_SWIGLU) {
      // 16-row interleave: even blocks gate, odd blocks up, same output columns
      const int blk = row >> 4, pr = blk >> 1;
      int j = tn * (TB / 2) + pr * 16 + (row & 15);
      j = min(j, a.N - 1);
      wr = (blk & 1) ? a.up_off + j : j;
    } else {
      wr = min(tn * TB + row, a.N - 1);
    }
    wsrc[i] = W + wr * a.ldw + col;
  }
  // activations: 2 chunks of 8 halves per plane per thread (4 threads per row);
  // rows past M read row M - 1: their outputs are never stored
  const f16_t* ahsrc[2];
  const f16_t* alsrc[2];
  int asoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i;
    const int row = c >> 2, col = (c & 3) * 8;
    asoff[i] = row * TLD + col;
    const int64_t off = (int64_t)min(tm * TB + row, a.M - 1) * a.lda + col;
    ahsrc[i] = (const f16_t*)a.A + off;
    alsrc[i] = (const f16_t*)a.A_lo + off;
  }
  // two register stages: the global loads of k step j are issued two steps
  // before step j is computed and are written to LDS at the end of step j - 1.
  // Every load is unconditional (indices are clamped instead) so that the
  // waits for one stage never cover the other stage's loads.
  u32x4 rw0[2], rh0[2], rl0[2], rw1[2], rh1[2], rl1[2];
  auto gload = [&](u32x4 (&rw)[2], u32x4 (&rh)[2], u32x4 (&rl)[2], int kt) {
    const int k0 = kt * TK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      rw[i] = *(const u32x4*)(wsrc[i] + k0);
      rh[i] = *(const u32x4*)(ahsrc[i] + k0);
      rl[i] = *(const u32x4*)(alsrc[i] + k0);
    }
  };
  auto sstore = [&](const u32x4 (&rw)[2], const u32x4 (&rh)[2], const u32x4 (&rl)[2], int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *(u32x4*)(&sw[buf][wsoff[i]]) = bf16x8_to_f16x8(rw[i]);
      *(u32x4*)(&sah[buf][asoff[i]]) = rh[i];
      *(u32x4*)(&sal[buf][asoff[i]]) = rl[i];
    }
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf) {
    u32x4 fw[4], fh[4], fl[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) fw[x] = *(const u32x4*)(&sw[buf][(wn + x * 16 + i16) * TLD + g * 8]);
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      fh[y] = *(const u32x4*)(&sah[buf][(wm + y * 16 + i16) * TLD + g * 8]);
      fl[y] = *(const u32x4*)(&sal[buf][(wm + y * 16 + i16) * TLD + g * 8]);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        acc[x][y] = mfma16(fw[x], fh[y], acc[x][y]);
        acc[x][y] = mfma16(fw[x], fl[y], acc[x][y]);
      }
  };

  const int nk = a.K / TK;
  const int kt0 = (int)((int64_t)nk * sp / splits), kt1 = (int)((int64_t)nk * (sp + 1) / splits);
  gload(rw0, rh0, rl0, kt0);
  sstore(rw0, rh0, rl0, 0);
  gload(rw1, rh1, rl1, min(kt0 + 1, kt1 - 1));
  __syncthreads();
  for (int kt = kt0; kt < kt1; kt += 2) {
    // even step: LDS buffer 0 holds step kt, stage 1 step kt + 1 (past the
    // end: a repeat of the last step, staged into a buffer nobody reads)
    gload(rw0, rh0, rl0, min(kt + 2, kt1 - 1));
    compute(0);
    sstore(rw1, rh1, rl1, 1);
    __syncthreads();
    if (kt + 1 >= kt1) break;
    // odd step: LDS buffer 1 holds step kt + 1, stage 0 step kt + 2
    gload(rw1, rh1, rl1, min(kt + 3, kt1 - 1));
    compute(1);
    sstore(rw0, rh0, rl0, 0);
    __syncthreads();
  }
  if (splits > 1) {
    // publish this split's partial tile; the last arrival sums all of them
    const int tile = tm * n_tn + tn;
    f32x4* mine = (f32x4*)(a.split_ws + ((int64_t)tile * splits + sp) * GEMM_TILE_FLOATS);
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) mine[(x * 4 + y) * 256 + tid] = acc[x][y];
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&a.split_cnt[tile], 1) == splits - 1;
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    // sum in split order (this work-group's own partial is read back too)
    const f32x4* all = (const f32x4*)(a.split_ws + (int64_t)tile * splits * GEMM_TILE_FLOATS) + tid;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) acc[x][y] = all[(x * 4 + y) * 256];
    for (int q = 1; q < splits; ++q) {
      const f32x4* pq = all + (int64_t)q * (GEMM_TILE_FLOATS / 4);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] += pq[(x * 4 + y) * 256];
    }
    if (tid == 0) a.split_cnt[tile] = 0;
  }
  // epilogue: acc[x][y] lane -> weight rows wn + 16x + 4g + r, activation row wm + 16y + i16
#pragma unroll
  for (int y = 0; y < 4; ++y) {
    const int m = tm * TB + wm + y * 16 + i16;
    if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int x = 0; x < 4; x += 2) {
        const int blk = (wn >> 4) + x;  // even block: gate; blk + 1: up
        const int n = tn * (TB / 2) + (blk >> 1) * 16 + 4 * g;
        epi4<EPI, true>(a, m, n, acc[x][y], acc[x + 1][y]);
      }
    } else {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int n = tn * TB + wn + x * 16 + 4 * g;
        epi4<EPI, true>(a, m, n, acc[x][y], acc[x][y]);
      }
    }
  }
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
  }
}

// One named kernel per projection and path, so that profiles attribute time
// to the projection (qkv, o, gate_up, down, lm_head) rather than to a shared
// template instance.
#define CAD_GEMM_KERNELS(NAME, EPI)                                                        \
  __global__ void __launch_bounds__(256, 2)                                                \
      k_gemm_##NAME(GemmArgs a, int n_tn, int n_tm, int splits) {                          \
    gemm_tiled_body<EPI>(a, n_tn, n_tm, splits);                                           \
  }                                                                                        \
  __global__ void __launch_bounds__(64 * SK_WAVES) k_gemv_##NAME(GemmArgs a) {             \
    gemm_skinny_body<EPI>(a);                                                              \
  }                                                                                        \
  __global__ void __launch_bounds__(256) k_gemm_f32_##NAME(GemmArgs a) { gemm_f32_body<EPI>(a); }

CAD_GEMM_KERNELS(qkv, EPI_STORE_F32)
CAD_GEMM_KERNELS(o, EPI_RESID)
CAD_GEMM_KERNELS(gate_up, EPI_SWIGLU)
CAD_GEMM_KERNELS(down, EPI_RESID)
CAD_GEMM_KERNELS(lm_head, EPI_STORE_F32)
#undef CAD_GEMM_KERNELS

typedef void (*TiledFn)(GemmArgs, int, int, int);
typedef void (*PlainFn)(GemmArgs);

template <int EPI>
static hipError_t launch_epi(int dtype, const GemmArgs& a, TiledFn tiled, PlainFn skinny, PlainFn f32,
                             hipStream_t s) {
  if (dtype == CAD_F32) {
    dim3 grid((a.N + 63) / 64, (a.M + 63) / 64);
    hipLaunchKernelGGL(f32, grid, dim3(256), 0, s, a);
  } else if (a.M <= 16) {
    hipLaunchKernelGGL(skinny, dim3((a.N + 15) / 16), dim3(64 * SK_WAVES), 0, s, a);
  } else {
    const int cols_per_tile = (EPI == EPI_SWIGLU) ? TB / 2 : TB;
    const int n_tn = (a.N + cols_per_tile - 1) / cols_per_tile, n_tm = (a.M + TB - 1) / TB;
    const int tiles = n_tn * n_tm, nk = a.K / TK;
    // split K while the tiles alone leave compute units idle (two
    // work-groups fit per CU), keeping at least 64 k steps of 32 per split
    int splits = 1;
    if (EPI != EPI_SWIGLU && a.split_ws && a.split_cnt)
      while (splits < 8 && tiles * splits * 2 <= GEMM_SPLIT_SLOTS && nk / (splits * 2) >= 64 &&
             (int64_t)tiles * splits * 2 * GEMM_TILE_FLOATS <= GEMM_SPLIT_FLOATS)
        splits *= 2;
    hipLaunchKernelGGL(tiled, dim3(tiles * splits), dim3(256), 0, s, a, n_tn, n_tm, splits);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, int role, const GemmArgs& a, hipStream_t s) {
  switch (role) {
    case GEMM_QKV: return launch_epi<EPI_STORE_F32>(dtype, a, k_gemm_qkv, k_gemv_qkv, k_gemm_f32_qkv, s);
    case GEMM_O: return launch_epi<EPI_RESID>(dtype, a, k_gemm_o, k_gemv_o, k_gemm_f32_o, s);
    case GEMM_GATE_UP:
      return launch_epi<EPI_SWIGLU>(dtype, a, k_gemm_gate_up, k_gemv_gate_up, k_gemm_f32_gate_up, s);
    case GEMM_DOWN: return launch_epi<EPI_RESID>(dtype, a, k_gemm_down, k_gemv_down, k_gemm_f32_down, s);
    default: return launch_epi<EPI_STORE_F32>(dtype, a, k_gemm_lm_head, k_gemv_lm_head, k_gemm_f32_lm_head, s);
  }
}

}  // namespace cad
