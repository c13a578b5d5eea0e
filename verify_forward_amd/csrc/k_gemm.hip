// Projection GEMMs of the splice path: C[m][n] = sum_k A[m][k] * W[n][k]
// (activations times nn.Linear weights, both K-contiguous), fp32 accumulate,
// with the consumer fused into the epilogue:
//   EPI_STORE_F32  C -> fp32 buffer (QKV projection, LM head)
//   EPI_RESID      x += C into the fp32 residual stream (O and down projections)
//   EPI_SWIGLU     silu(C_gate) * C_up -> activation (gate/up projection)
//
// bf16 models use the gfx950 matrix cores in half precision
// (v_mfma_f32_16x16x32_f16): weights stay bf16 in HBM and are widened to half
// in registers (exact in half's normal range), activations arrive as half,
// so the only rounding left at a projection input is half's 11-bit mantissa
// instead of bf16's 8.  The MFMA is issued with the weight tile as its first
// operand and the activations as the second, so each lane ends up holding four consecutive output columns of one
// row (C^T layout: lane l, register r -> column 4*(l/16)+r, row l%16).
//   * skinny (M <= 16): weight-streaming.  A work-group owns 16 output
//     columns (32 weight rows for SWIGLU); its four waves split K and are
//     reduced through LDS in a fixed order.  Every lane loads 32 contiguous
//     bytes of a weight row per 64-wide k step straight into registers.
//   * tiled (M > 16): 128x128 output tile per 256-thread work-group, K in
//     steps of 64 staged through double-buffered LDS.  When the output has
//     too few tiles to occupy the 256 compute units, K is split over up to
//     eight work-groups per tile; each writes its fp32 partial tile to the
//     workspace and the last to arrive (per-tile counter) sums the partials
//     in split order and runs the epilogue, so results do not depend on
//     scheduling.  The global loads run two k steps ahead of the matrix
//     cores (two register stages in front of the LDS double buffer).
// fp32 (the small reference-shape path) uses a plain LDS-tiled VALU kernel.
#include "cad_internal.h"

namespace cad {

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Apply the epilogue to four consecutive output columns n .. n+3 of row m.
// For SWIGLU `c` holds the gate values and `cu` the matching up values.
template <int EPI, typename TA>
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
  } else {
    TA* o = (TA*)a.out_act + (int64_t)m * a.N + n;
    for (int r = 0; r < 4; ++r)
      if (n + r < a.N) o[r] = from_f<TA>(silu_mul(c[r], cu[r]));
  }
}

// ---------------------------------------------------------------------------
// bf16 skinny: M <= 16
// ---------------------------------------------------------------------------
constexpr int SK_WAVES = 4;

template <int EPI>
__global__ void __launch_bounds__(64 * SK_WAVES)
k_gemm_skinny(GemmArgs a) {
  constexpr int NB = (EPI == EPI_SWIGLU) ? 2 : 1;  // 16-row weight blocks per work-group
  __shared__ f32x4 part[SK_WAVES][NB][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, i16 = lane & 15;
  const int n0 = blockIdx.x * 16;
  const f16_t* A = (const f16_t*)a.A;
  const bf16_t* W = (const bf16_t*)a.W;
  // this lane's weight rows (clamped: columns past N are computed and dropped)
  const int ncol = min(n0 + i16, a.N - 1);
  const bf16_t* wrow[NB];
  wrow[0] = W + (int64_t)ncol * a.ldw;
  if (NB == 2) wrow[NB - 1] = W + (a.up_off + ncol) * a.ldw;
  const bool arow_ok = i16 < a.M;
  const f16_t* arow = A + (int64_t)(arow_ok ? i16 : 0) * a.lda;
  // k split across waves in units of 64
  const int kp_total = a.K / 64;
  const int kp0 = (kp_total * wave) / SK_WAVES, kp1 = (kp_total * (wave + 1)) / SK_WAVES;
  f32x4 acc[NB];
  for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 zero = {0u, 0u, 0u, 0u};
  constexpr int U = 4;
  int kp = kp0;
  for (; kp + U <= kp1; kp += U) {
    u32x4 wv[NB][U][2], av[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (kp + u) * 64 + g * 16;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const u32x4* p = (const u32x4*)(wrow[b] + k);
        wv[b][u][0] = __builtin_nontemporal_load(p);
        wv[b][u][1] = __builtin_nontemporal_load(p + 1);
      }
      const u32x4* q = (const u32x4*)(arow + k);
      av[u][0] = arow_ok ? q[0] : zero;
      av[u][1] = arow_ok ? q[1] : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        acc[b] = mfma16(bf16x8_to_f16x8(wv[b][u][0]), av[u][0], acc[b]);
        acc[b] = mfma16(bf16x8_to_f16x8(wv[b][u][1]), av[u][1], acc[b]);
      }
  }
  for (; kp < kp1; ++kp) {
    const int k = kp * 64 + g * 16;
    u32x4 a0 = zero, a1 = zero;
    if (arow_ok) { a0 = ((const u32x4*)(arow + k))[0]; a1 = ((const u32x4*)(arow + k))[1]; }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const u32x4* p = (const u32x4*)(wrow[b] + k);
      acc[b] = mfma16(bf16x8_to_f16x8(p[0]), a0, acc[b]);
      acc[b] = mfma16(bf16x8_to_f16x8(p[1]), a1, acc[b]);
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
    epi4<EPI, f16_t>(a, i16, n0 + 4 * g, s[0], s[NB - 1]);
  }
}

// ---------------------------------------------------------------------------
// bf16 tiled: 128 (weight rows) x 128 (activation rows) per work-group
// ---------------------------------------------------------------------------
constexpr int TB = 128, TK = 64, TPAD = 8, TLD = TK + TPAD;

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
__global__ void __launch_bounds__(256, 2)
k_gemm_tiled(GemmArgs a, int n_tn, int n_tm, int splits) {
  __shared__ __attribute__((aligned(16))) f16_t sw[2][TB * TLD];
  __shared__ __attribute__((aligned(16))) f16_t sa[2][TB * TLD];
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, i16 = lane & 15;
  const int wn = (wave & 1) * 64;   // wave's offset in the weight-row dim of the tile
  const int wm = (wave >> 1) * 64;  // wave's offset in the activation-row dim
  int tn, tm, sp;
  gemm_tile_of(n_tn, n_tm, tn, tm, sp);
  const f16_t* A = (const f16_t*)a.A;
  const bf16_t* W = (const bf16_t*)a.W;

  // global -> LDS assignment: 4 chunks of 8 bf16 per thread per operand
  const bf16_t* wsrc[4];
  const f16_t* asrc[4];
  int soff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int row = c >> 3, col = (c & 7) * 8;
    soff[i] = row * TLD + col;
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
    // activation rows past M read row M - 1: their outputs are never stored
    asrc[i] = A + (int64_t)min(tm * TB + row, a.M - 1) * a.lda + col;
  }
  // two register stages: the global loads of k step j are issued two steps
  // before step j is computed and are written to LDS at the end of step j - 1.
  // Every load is unconditional (indices are clamped instead) so that the
  // waits for one stage never cover the other stage's loads.
  u32x4 rw0[4], ra0[4], rw1[4], ra1[4];
  auto gload = [&](u32x4 (&rw)[4], u32x4 (&ra)[4], int kt) {
    const int k0 = kt * TK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rw[i] = *(const u32x4*)(wsrc[i] + k0);
      ra[i] = *(const u32x4*)(asrc[i] + k0);
    }
  };
  auto sstore = [&](const u32x4 (&rw)[4], const u32x4 (&ra)[4], int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(u32x4*)(&sw[buf][soff[i]]) = bf16x8_to_f16x8(rw[i]);
      *(u32x4*)(&sa[buf][soff[i]]) = ra[i];
    }
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < TK / 32; ++ks) {
      u32x4 fw[4], fa[4];
#pragma unroll
      for (int x = 0; x < 4; ++x)
        fw[x] = *(const u32x4*)(&sw[buf][(wn + x * 16 + i16) * TLD + ks * 32 + g * 8]);
#pragma unroll
      for (int y = 0; y < 4; ++y)
        fa[y] = *(const u32x4*)(&sa[buf][(wm + y * 16 + i16) * TLD + ks * 32 + g * 8]);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
          acc[x][y] = mfma16(fw[x], fa[y], acc[x][y]);
    }
  };

  const int nk = a.K / TK;
  const int kt0 = (int)((int64_t)nk * sp / splits), kt1 = (int)((int64_t)nk * (sp + 1) / splits);
  gload(rw0, ra0, kt0);
  sstore(rw0, ra0, 0);
  gload(rw1, ra1, min(kt0 + 1, kt1 - 1));
  __syncthreads();
  for (int kt = kt0; kt < kt1; kt += 2) {
    // even step: LDS buffer 0 holds step kt, stage 1 step kt + 1 (past the
    // end: a repeat of the last step, staged into a buffer nobody reads)
    gload(rw0, ra0, min(kt + 2, kt1 - 1));
    compute(0);
    sstore(rw1, ra1, 1);
    __syncthreads();
    if (kt + 1 >= kt1) break;
    // odd step: LDS buffer 1 holds step kt + 1, stage 0 step kt + 2
    gload(rw1, ra1, min(kt + 3, kt1 - 1));
    compute(1);
    sstore(rw0, ra0, 0);
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
        epi4<EPI, f16_t>(a, m, n, acc[x][y], acc[x + 1][y]);
      }
    } else {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int n = tn * TB + wn + x * 16 + 4 * g;
        epi4<EPI, f16_t>(a, m, n, acc[x][y], acc[x][y]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 VALU path: 64x64 tile, 256 threads, 4x4 outputs each
// ---------------------------------------------------------------------------
template <int EPI>
__global__ void __launch_bounds__(256)
k_gemm_f32(GemmArgs a) {
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
    epi4<EPI, float>(a, m, n0 + tx * 4, c, cu);
  }
}

template <int EPI>
static hipError_t launch_epi(int dtype, const GemmArgs& a, hipStream_t s) {
  if (dtype == CAD_F32) {
    dim3 grid((a.N + 63) / 64, (a.M + 63) / 64);
    hipLaunchKernelGGL(k_gemm_f32<EPI>, grid, dim3(256), 0, s, a);
  } else if (a.M <= 16) {
    hipLaunchKernelGGL(k_gemm_skinny<EPI>, dim3((a.N + 15) / 16), dim3(64 * SK_WAVES), 0, s, a);
  } else {
    const int cols_per_tile = (EPI == EPI_SWIGLU) ? TB / 2 : TB;
    const int n_tn = (a.N + cols_per_tile - 1) / cols_per_tile, n_tm = (a.M + TB - 1) / TB;
    const int tiles = n_tn * n_tm, nk = a.K / TK;
    // split K while the tiles alone leave compute units idle (two
    // work-groups fit per CU), keeping at least 32 k steps per split
    int splits = 1;
    if (EPI != EPI_SWIGLU && a.split_ws && a.split_cnt)
      while (splits < 8 && tiles * splits * 2 <= GEMM_SPLIT_SLOTS && nk / (splits * 2) >= 32) splits *= 2;
    hipLaunchKernelGGL(k_gemm_tiled<EPI>, dim3(tiles * splits), dim3(256), 0, s, a, n_tn, n_tm, splits);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, int epi, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_STORE_F32: return launch_epi<EPI_STORE_F32>(dtype, a, s);
    case EPI_RESID: return launch_epi<EPI_RESID>(dtype, a, s);
    default: return launch_epi<EPI_SWIGLU>(dtype, a, s);
  }
}

}  // namespace cad
