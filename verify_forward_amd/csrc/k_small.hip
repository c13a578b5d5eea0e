// Row-wise kernels of the splice path: embedding gather, RMSNorm, rotary
// positions + KV append, masked argmax, acceptance scan and the suffix-match
// proposal.  All are bandwidth- or latency-bound; one work-group per row.
#include "cad_internal.h"

namespace cad {

constexpr int ROW_THREADS = 256;

__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  const int nw = blockDim.x >> 6;
  for (int i = 0; i < nw; ++i) t += red[i];  // fixed order: reproducible
  __syncthreads();
  return t;
}

// ---------------------------------------------------------------------------
// embedding gather: x[r] = E[token[r]] widened to fp32 (the residual stream)
// ---------------------------------------------------------------------------
template <typename T>
__global__ void k_embed(const T* __restrict__ table, int vocab, int d, const int32_t* __restrict__ tok,
                        float* __restrict__ x, int32_t* status) {
  const int r = blockIdx.x;
  const int t = tok[r];
  const bool ok = t >= 0 && t < vocab;
  if (!ok && threadIdx.x == 0 && status) atomicOr(status, (int32_t)CAD_DEV_BAD_TOKEN);
  const T* src = table + (int64_t)(ok ? t : 0) * d;
  float* dst = x + (int64_t)r * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) dst[i] = ok ? to_f<T>(src[i]) : 0.f;
}

hipError_t launch_embed(int dtype, const void* table, int vocab, int d, const int32_t* tokens,
                        int rows, float* x, int32_t* status, hipStream_t s) {
  if (dtype == CAD_BF16)
    hipLaunchKernelGGL(k_embed<bf16_t>, dim3(rows), dim3(ROW_THREADS), 0, s,
                       (const bf16_t*)table, vocab, d, tokens, x, status);
  else
    hipLaunchKernelGGL(k_embed<float>, dim3(rows), dim3(ROW_THREADS), 0, s, (const float*)table,
                       vocab, d, tokens, x, status);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RMSNorm: out[r] = x[r] / sqrt(mean(x[r]^2) + eps) * g: fp32 for fp32
// models, split into bf16 hi / lo planes (the next projection's operands)
// for bf16 models
// ---------------------------------------------------------------------------
template <typename T, bool SPLIT, int V4, int NT>
__global__ void __launch_bounds__(NT) k_rmsnorm(float* __restrict__ x, const float* __restrict__ x_part,
                                                int n_part, int rows, const T* __restrict__ g, int d,
                                                float eps, void* __restrict__ out, void* __restrict__ out_lo) {
  // each of the NT threads keeps up to V4 groups of four elements in
  // registers: one pass over x, all loads issued before the reduction.
  // Pending k-split partial sums of the projection that last wrote x
  // ([n_part][rows][d], up to one plane per 512 k of the projection) are added
  // first, in split order, and x is written back.
  __shared__ float red[NT / 64];
  const int r = blockIdx.x;
  float* xr = x + (int64_t)r * d;
  const int n4 = d / 4;
  f32x4 v[V4], gv[V4];
  float ss = 0.f;
  // x and the gain are both loaded up front (the gain does not wait for
  // the reduction)
#pragma unroll
  for (int j = 0; j < V4; ++j) {
    const int i4 = threadIdx.x + j * NT;
    v[j] = i4 < n4 ? *(const f32x4*)(xr + 4 * i4) : f32x4{0.f, 0.f, 0.f, 0.f};
    const int c4 = min(i4, n4 - 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) gv[j][e] = to_f<T>(g[4 * c4 + e]);
  }
  if (n_part > 0) {
    // PB partial planes per batch, all their loads in flight together
    // (indices clamped; the clamped repeats are not added)
    constexpr int PB = NT >= 1024 ? 16 / V4 : (V4 <= 2 ? 8 : 16 / V4);
    for (int sp = 0; sp < n_part; sp += PB) {
      f32x4 t[PB][V4];
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        const float* pr = x_part + ((int64_t)min(sp + u, n_part - 1) * rows + r) * d;
#pragma unroll
        for (int j = 0; j < V4; ++j) {
          const int i4 = min((int)threadIdx.x + j * NT, n4 - 1);
          t[u][j] = *(const f32x4*)(pr + 4 * i4);
        }
      }
#pragma unroll
      for (int u = 0; u < PB; ++u)
        if (sp + u < n_part)
#pragma unroll
          for (int j = 0; j < V4; ++j) v[j] += t[u][j];
    }
#pragma unroll
    for (int j = 0; j < V4; ++j) {
      const int i4 = threadIdx.x + j * NT;
      if (i4 < n4) *(f32x4*)(xr + 4 * i4) = v[j];
    }
  }
#pragma unroll
  for (int j = 0; j < V4; ++j) ss += v[j][0] * v[j][0] + v[j][1] * v[j][1] + v[j][2] * v[j][2] + v[j][3] * v[j][3];
  ss = block_sum(ss, red);
  const float rs = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int j = 0; j < V4; ++j) {
    const int i4 = threadIdx.x + j * NT;
    if (i4 >= n4) continue;
    const int i = 4 * i4;
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = v[j][e] * rs * gv[j][e];
    if (SPLIT) {
      bf16_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) split_bf16(y[e], hi[e], lo[e]);
      *(u32x2*)((bf16_t*)out + (int64_t)r * d + i) = u32x2{hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16)};
      *(u32x2*)((bf16_t*)out_lo + (int64_t)r * d + i) =
          u32x2{lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16)};
    } else {
      *(f32x4*)((float*)out + (int64_t)r * d + i) = f32x4{y[0], y[1], y[2], y[3]};
    }
  }
}

hipError_t launch_rmsnorm(int dtype, float* x, const float* x_part, int n_part, const void* gain, int rows, int d,
                          float eps, void* out, void* out_lo, hipStream_t s) {
  // few rows of 4096 and more (short spans, whose projections leave up to
  // one partial plane per 512 k): 1024 threads, one or two groups
  // of four each, so that 16 / V4 planes are in flight at once; else 256
  const int nt = (d >= 4096 && rows <= 64) ? 1024 : ROW_THREADS;
  const int v4 = (d / 4 + nt - 1) / nt;
  if (d % 4 != 0 || v4 > 8 || (n_part > 0 && !x_part)) return hipErrorInvalidValue;
#define CAD_RMS(V, NT)                                                                                     \
  if (v4 <= V && nt == NT) {                                                                               \
    if (dtype == CAD_BF16)                                                                                 \
      hipLaunchKernelGGL((k_rmsnorm<bf16_t, true, V, NT>), dim3(rows), dim3(NT), 0, s, x, x_part, n_part,  \
                         rows, (const bf16_t*)gain, d, eps, out, out_lo);                                  \
    else                                                                                                   \
      hipLaunchKernelGGL((k_rmsnorm<float, false, V, NT>), dim3(rows), dim3(NT), 0, s, x, x_part, n_part,  \
                         rows, (const float*)gain, d, eps, out, out_lo);                                   \
    return hipGetLastError();                                                                              \
  }
  CAD_RMS(1, 256) CAD_RMS(2, 256) CAD_RMS(4, 256) CAD_RMS(8, 256)
  CAD_RMS(1, 1024) CAD_RMS(2, 1024) CAD_RMS(4, 1024) CAD_RMS(8, 1024)
#undef CAD_RMS
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// RMSNorm for a few rows (the weight-streaming projections that follow
// normalise while they stage their activations): x += the pending k-split
// partial planes, one 256-element slice per work-group (so a single row is
// spread over d / 256 compute units), and the slice's sum of squares to
// ss[row][slice].  The consumer forms 1 / sqrt(sum(ss[row]) / d + eps) from
// the slice sums in slice order.
// ---------------------------------------------------------------------------
constexpr int RMS_SLICE = 256;

__global__ void __launch_bounds__(64) k_rms_slices(float* __restrict__ x, const float* __restrict__ x_part,
                                                   int n_part, int rows, int d, float* __restrict__ ss) {
  const int r = blockIdx.x, sl = blockIdx.y;
  const int n4 = d / 4;
  const int i4 = sl * (RMS_SLICE / 4) + threadIdx.x;
  const int c4 = min(i4, n4 - 1);
  float* xr = x + (int64_t)r * d;
  f32x4 v = *(const f32x4*)(xr + 4 * c4);
  // PB planes in flight at once (clamped repeats are not added)
  constexpr int PB = 8;
  for (int sp = 0; sp < n_part; sp += PB) {
    f32x4 t[PB];
#pragma unroll
    for (int u = 0; u < PB; ++u) t[u] = *(const f32x4*)(x_part + ((int64_t)min(sp + u, n_part - 1) * rows + r) * d + 4 * c4);
#pragma unroll
    for (int u = 0; u < PB; ++u)
      if (sp + u < n_part) v += t[u];
  }
  const bool ok = i4 < n4;
  if (n_part > 0 && ok) *(f32x4*)(xr + 4 * i4) = v;
  float q = ok ? v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3] : 0.f;
  for (int o = 32; o > 0; o >>= 1) q += __shfl_xor(q, o);
  if (threadIdx.x == 0) ss[(int64_t)r * gridDim.y + sl] = q;
}

int rms_slices(int d) { return (d + RMS_SLICE - 1) / RMS_SLICE; }

hipError_t launch_rms_slices(float* x, const float* x_part, int n_part, int rows, int d, float* ss, hipStream_t s) {
  if (d % 4 != 0 || rows < 1 || (n_part > 0 && !x_part)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_rms_slices, dim3(rows, rms_slices(d)), dim3(RMS_SLICE / 4), 0, s, x, x_part, n_part, rows, d, ss);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// rotary positions on q and k (half-split pairs, angle pos * freq[i] formed
// and reduced in fp64), q to the attention operand buffer (type TQ), k and v appended to
// the paged cache (type T) at the row's absolute position.  Rows at or beyond
// *write_limit do not touch the cache.  bf16 models also keep every row's k
// and v at half precision in the span workspace (kv.span_k / kv.span_v),
// which attention reads for this call's own keys.
// One work-group per row and group of heads: with gridDim.y == 1 the whole
// row, with gridDim.y == hkv one KV group (its G query heads, its k head and
// its v head), so that a few rows still spread their staging loads (the
// k-split partials of the QKV projection) over many compute units.
// ---------------------------------------------------------------------------
constexpr int ROPE_MAX_HALF = 128;  // head_dim up to 256
constexpr int ROPE_THREADS = 512;

template <typename T, typename TQ>
__global__ void __launch_bounds__(ROPE_THREADS) k_rope_append(const float* __restrict__ qkv, const float* __restrict__ qkv_part, int n_part,
                              int rows, int hq, int hkv, int hd,
                              const double* __restrict__ freq, RowMap rm, KVView kv,
                              const int32_t* write_limit, TQ* __restrict__ q_out, TQ* __restrict__ q_lo,
                              int32_t* status) {
  const int r = blockIdx.x;
  const int b = row_seq(rm, r);
  const int local = r - rm.start[b];
  const int64_t pos = rm.L[b] + local;
  const int half = hd / 2;
  const int width = (hq + 2 * hkv) * hd;
  // this work-group's heads: query heads [qh0, qh0 + nq), kv heads [kh0, kh0 + nk)
  const bool grouped = gridDim.y > 1;
  const int nq = grouped ? hq / hkv : hq, nk = grouped ? 1 : hkv;
  const int qh0 = grouped ? blockIdx.y * nq : 0, kh0 = grouped ? blockIdx.y : 0;
  // independent loads first: this row's cache block and its rotation
  // frequency (one pair per thread)
  bool write_kv = write_limit == nullptr || local < *write_limit;
  const int64_t blk = write_kv ? kv.table[(int64_t)b * kv.max_blocks + pos / CAD_KV_BLOCK] : 0;
  const double fr = (int)threadIdx.x < half ? freq[threadIdx.x] : 0.0;
  // the row's projection output for these heads, staged in LDS as
  // [q heads][k heads][v heads] x hd: the stored values, or the sum of the
  // k-split partials [n_part][rows][width] in split order
  extern __shared__ float srow[];
  {
    const float* src = n_part == 0 ? qkv + (int64_t)r * width : qkv_part + (int64_t)r * width;
    const int64_t plane = (int64_t)rows * width;
    const int nqc = nq * hd, nkc = nk * hd;  // staged columns of q, and of k (and of v)
    const int staged = nqc + 2 * nkc;
    // staged column j -> projection column (the three runs are contiguous)
    auto src_col = [&](int j) {
      return j < nqc ? qh0 * hd + j
                     : (j < nqc + nkc ? (hq + kh0) * hd + (j - nqc) : (hq + hkv + kh0) * hd + (j - nqc - nkc));
    };
    // RV 16-byte pieces per thread in flight at once (indices clamped; the
    // clamped repeats are not stored); partial planes added in split order.
    // hd is a multiple of 4, so a 4-column piece never straddles two runs.
    const int n4 = (hd % 4 == 0) ? staged / 4 : 0;
    constexpr int RV = 4;
    for (int base = 0; base < n4; base += RV * ROPE_THREADS) {
      f32x4 v[RV];
      int col[RV];
#pragma unroll
      for (int u = 0; u < RV; ++u) {
        col[u] = src_col(4 * min(base + (int)threadIdx.x + u * ROPE_THREADS, n4 - 1));
        v[u] = *(const f32x4*)(src + col[u]);
      }
      for (int sp = 1; sp < n_part; ++sp) {
        f32x4 t[RV];
#pragma unroll
        for (int u = 0; u < RV; ++u) t[u] = *(const f32x4*)(src + sp * plane + col[u]);
#pragma unroll
        for (int u = 0; u < RV; ++u) v[u] += t[u];
      }
#pragma unroll
      for (int u = 0; u < RV; ++u) {
        const int i4 = base + (int)threadIdx.x + u * ROPE_THREADS;
        if (i4 < n4) *(f32x4*)(srow + 4 * i4) = v[u];
      }
    }
    for (int j = 4 * n4 + threadIdx.x; j < staged; j += blockDim.x) {
      const int c = src_col(j);
      float v = src[c];
      for (int sp = 1; sp < n_part; ++sp) v += src[sp * plane + c];
      srow[j] = v;
    }
  }
  auto ld = [&](int i) { return srow[i]; };
  if (write_kv && (blk < 0 || blk >= kv.num_blocks)) {
    if (threadIdx.x == 0 && status) atomicOr(status, (int32_t)CAD_DEV_BAD_BLOCK);
    write_kv = false;
  }
  const int slot = (int)(pos % CAD_KV_BLOCK);
  T* kc = (T*)kv.k;
  T* vc = (T*)kv.v;
  const int64_t wrow = rm.pstart[b] + local;  // span workspace row
  f16_t* sk = kv.span_k ? kv.span_k + wrow * hkv * hd : nullptr;
  // the row's rotation, one (cos, sin) per pair, in LDS
  __shared__ float2 rot[ROPE_MAX_HALF];
  if ((int)threadIdx.x < half) {
    const int i = threadIdx.x;
    // angle pos * freq[i] in fp64, reduced by a multiple of 2 pi (2 pi split
    // into a double and its remainder, Cody-Waite) to |r| <= pi, whose sine
    // and cosine single precision takes on its fast path
    const double ang = (double)pos * fr;
    const double k = rint(ang * 0.15915494309189535);           // 1 / (2 pi)
    double r = fma(-k, 6.283185307179586, ang);                  // 2 pi, high part
    r = fma(-k, 2.4492935982947064e-16, r);                      // 2 pi - high part
    float sn, cs;
    sincosf((float)r, &sn, &cs);
    rot[i] = float2{cs, sn};
  }
  __syncthreads();
  // rotations: q heads then k heads (staged order), one (head, pair) per item
  const int n_rot = (nq + nk) * half;
  for (int it = threadIdx.x; it < n_rot; it += blockDim.x) {
    const int hs = it / half, i = it % half;
    const float c = rot[i].x, s = rot[i].y;
    const float a = ld(hs * hd + i), bb = ld(hs * hd + i + half);
    const float ra = a * c - bb * s, rb = a * s + bb * c;
    if (hs < nq) {
      const int h = qh0 + hs;
      TQ* qo = q_out + ((int64_t)r * hq + h) * hd;
      qo[i] = from_f<TQ>(ra);
      qo[i + half] = from_f<TQ>(rb);
      if (q_lo) {  // half-precision remainder plane: q = hi + lo to ~2^-22
        TQ* ql = q_lo + ((int64_t)r * hq + h) * hd;
        ql[i] = from_f<TQ>(ra - to_f<TQ>(qo[i]));
        ql[i + half] = from_f<TQ>(rb - to_f<TQ>(qo[i + half]));
      }
    } else {
      const int g = kh0 + hs - nq;
      if (write_kv) {
        T* kd = kc + ((blk * hkv + g) * CAD_KV_BLOCK + slot) * hd;
        kd[i] = from_f<T>(ra);
        kd[i + half] = from_f<T>(rb);
      }
      if (sk) {
        sk[g * hd + i] = f2h(ra);
        sk[g * hd + i + half] = f2h(rb);
      }
    }
  }
  for (int it = threadIdx.x; it < nk * hd; it += blockDim.x) {
    const int g = kh0 + it / hd, dd = it % hd;
    const float vv = ld((nq + nk) * hd + it);
    if (write_kv) vc[((blk * hkv + g) * hd + dd) * CAD_KV_BLOCK + slot] = from_f<T>(vv);
    if (kv.span_v) kv.span_v[((int64_t)g * hd + dd) * kv.span_cap + wrow] = f2h(vv);
  }
}

// rows at most this many: one work-group per (row, KV group)
constexpr int ROPE_GROUPED_MAX_ROWS = 64;

hipError_t launch_rope_append(int dtype, const float* qkv, const float* qkv_part, int n_part, int rows, int hq,
                              int hkv, int hd, const double* freq, const RowMap& rm, KVView kv,
                              const int32_t* write_limit, void* q_out, void* q_lo, int32_t* status,
                              hipStream_t s) {
  const bool grouped = rows <= ROPE_GROUPED_MAX_ROWS && hkv > 1;
  const int heads = grouped ? hq / hkv + 2 : hq + 2 * hkv;
  const size_t lds = (size_t)heads * hd * sizeof(float);
  if (hd / 2 > ROPE_MAX_HALF || hd / 2 > ROPE_THREADS || (n_part > 0 && !qkv_part) || lds > 65536)
    return hipErrorInvalidValue;
  const dim3 grid(rows, grouped ? hkv : 1);
  if (dtype == CAD_BF16)
    hipLaunchKernelGGL((k_rope_append<bf16_t, f16_t>), grid, dim3(ROPE_THREADS), lds, s, qkv, qkv_part, n_part,
                       rows, hq, hkv, hd, freq, rm, kv, write_limit, (f16_t*)q_out, (f16_t*)q_lo, status);
  else
    hipLaunchKernelGGL((k_rope_append<float, float>), grid, dim3(ROPE_THREADS), lds, s, qkv, qkv_part, n_part,
                       rows, hq, hkv, hd, freq, rm, kv, write_limit, (float*)q_out, (float*)nullptr, status);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// masked argmax per row over fp32 logits: lowest id among equal maxima,
// -1 (and CAD_DEV_EMPTY_MASK) when the row allows nothing
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return bi < 0 || v > bv || (v == bv && i < bi);
}

constexpr int ARGMAX_THREADS = 1024;

// One work-group per row; each thread takes whole 32-token mask words: the
// word and its 32 logits (eight 16-byte loads, all in flight together) are
// read unconditionally (indices clamped to the row) and the allowed ids are
// compared in registers, in increasing id order.
__global__ void __launch_bounds__(ARGMAX_THREADS) k_argmax(const float* __restrict__ logits, int vocab,
                                                           const uint32_t* __restrict__ mask,
                                                           int32_t* __restrict__ out, int32_t* status) {
  __shared__ float sv[ARGMAX_THREADS / 64];
  __shared__ int si[ARGMAX_THREADS / 64];
  const int r = blockIdx.x;
  const float* lg = logits + (int64_t)r * vocab;
  const int words = (vocab + 31) / 32;
  const bool vec = (vocab & 3) == 0;  // rows 16-byte aligned: vector loads
  float bv = 0.f;
  int bi = -1;
  for (int w = threadIdx.x; w < words; w += blockDim.x) {
    const uint32_t bits = mask ? mask[(int64_t)r * words + w] : 0xFFFFFFFFu;
    float x[32];
    if (vec) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int v4 = min(w * 8 + j, vocab / 4 - 1);
        const f32x4 t = *(const f32x4*)(lg + 4 * v4);
        x[4 * j] = t[0], x[4 * j + 1] = t[1], x[4 * j + 2] = t[2], x[4 * j + 3] = t[3];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) x[j] = lg[min(w * 32 + j, vocab - 1)];
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int v = w * 32 + j;
      if (((bits >> j) & 1u) && v < vocab && better(x[j], v, bv, bi)) { bv = x[j]; bi = v; }
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int oi = __shfl_xor(bi, o);
    if (oi >= 0 && better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) { sv[wv] = bv; si[wv] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i)
      if (si[i] >= 0 && better(sv[i], si[i], bv, bi)) { bv = sv[i]; bi = si[i]; }
    out[r] = bi;
    if (bi < 0 && status) atomicOr(status, (int32_t)CAD_DEV_EMPTY_MASK);
  }
}

hipError_t launch_argmax(const float* logits, int rows, int vocab, const uint32_t* mask,
                         int32_t* out, int32_t* status, hipStream_t s) {
  if (vocab <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_argmax, dim3(rows), dim3(ARGMAX_THREADS), 0, s, logits, vocab, mask, out, status);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// acceptance: COMMIT -> N; VERIFY -> 1 + leading j >= 1 with a[j-1] == s[j].
// `limit` (device, optional) caps the rows examined (the screening survivors).
// ---------------------------------------------------------------------------
__global__ void k_accept(const int32_t* __restrict__ a, const int32_t* __restrict__ span, RowMap rm,
                         int mode, const int32_t* limit, int32_t* __restrict__ accepted) {
  const int b = threadIdx.x;
  if (b >= rm.n_seq) return;
  const int s0 = rm.start[b];
  int n = rm.start[b + 1] - s0;
  if (limit) n = min(n, max(1, *limit));
  int acc = n;
  if (mode == CAD_VERIFY) {
    acc = 1;
    while (acc < n && a[s0 + acc - 1] == span[s0 + acc]) ++acc;
  }
  accepted[b] = acc;
}

hipError_t launch_accept(const int32_t* argmax, const int32_t* span, const RowMap& rm, int mode,
                         const int32_t* limit, int32_t* accepted, hipStream_t s) {
  hipLaunchKernelGGL(k_accept, dim3(1), dim3(64), 0, s, argmax, span, rm, mode, limit, accepted);
  return hipGetLastError();
}

__global__ void k_fill_i32(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_i32, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

__global__ void k_mask_rows(int32_t* a, int rows, const int32_t* limit) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < rows && i >= *limit) a[i] = -1;
}

hipError_t launch_mask_rows(int32_t* argmax, int rows, const int32_t* limit, hipStream_t s) {
  hipLaunchKernelGGL(k_mask_rows, dim3((rows + 255) / 256), dim3(256), 0, s, argmax, rows, limit);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// suffix-match proposal: one work-group scans every start p for each suffix
// length n (max_n down to min_n) and keeps the largest matching p
// ---------------------------------------------------------------------------
constexpr int SUFFIX_THREADS = 1024;

__global__ void __launch_bounds__(SUFFIX_THREADS)
k_suffix_match(const int32_t* __restrict__ x, int64_t T, int max_n, int min_n, int K,
               int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_len,
               int64_t* __restrict__ out_pos) {
  __shared__ int32_t suf[64];
  __shared__ long long red[SUFFIX_THREADS / 64];
  __shared__ long long found;
  const int top = (int)((T - 1 < (int64_t)max_n) ? (T - 1) : max_n);
  if (threadIdx.x == 0) found = -1;
  __syncthreads();
  for (int n = top; n >= min_n && n >= 1; --n) {
    if (threadIdx.x < n) suf[threadIdx.x] = x[T - n + threadIdx.x];
    __syncthreads();
    long long best = -1;
    const int64_t last = T - 1 - n;  // p + n <= T - 1
    for (int64_t p = threadIdx.x; p <= last; p += blockDim.x) {
      bool m = true;
      for (int j = 0; j < n && m; ++j) m = x[p + j] == suf[j];
      if (m && p > best) best = p;
    }
    for (int o = 32; o > 0; o >>= 1) {
      const long long ob = __shfl_xor(best, o);
      best = ob > best ? ob : best;
    }
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
      long long b = -1;
      for (int i = 0; i < SUFFIX_THREADS / 64; ++i) b = red[i] > b ? red[i] : b;
      if (b >= 0) found = b + n;
    }
    __syncthreads();
    if (found >= 0) break;
  }
  const long long start = found;
  if (start < 0) {
    if (threadIdx.x == 0) { *out_len = 0; *out_pos = -1; }
    return;
  }
  const long long end = (start + K < T) ? start + K : T;
  const int len = (int)(end - start);
  for (int j = threadIdx.x; j < len; j += blockDim.x) out_tokens[j] = x[start + j];
  if (threadIdx.x == 0) { *out_len = len; *out_pos = start; }
}

hipError_t launch_suffix_match(const int32_t* tokens, int64_t T, int max_n, int min_n, int K,
                               int32_t* out_tokens, int32_t* out_len, int64_t* out_pos,
                               hipStream_t s) {
  hipLaunchKernelGGL(k_suffix_match, dim3(1), dim3(SUFFIX_THREADS), 0, s, tokens, T, max_n, min_n, K,
                     out_tokens, out_len, out_pos);
  return hipGetLastError();
}

}  // namespace cad
