// Row-wise kernels of the splice path: embedding gather, RMSNorm, rotary
// positions + KV append, the decision step (masked argmax from the LM head's
// candidates, acceptance scan) and the suffix-match proposal.  All are
// bandwidth- or latency-bound.
#include "cad_internal.h"
#include "suffix_match.h"

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
// pipeline tick of a looped decoder: each row's residual stream is the
// embedding of its token on its group's first application of the shared
// block, and the state saved by the previous tick afterwards; after the tick
// every row's stream (with the pending k-split partials of the last
// projection added in split order) is saved again
// ---------------------------------------------------------------------------
template <typename T>
__global__ void k_loop_load(const T* __restrict__ table, int vocab, int d, const int32_t* __restrict__ tok,
                            const float* __restrict__ state, RowMap rm, StateMap sm, float* __restrict__ x,
                            int32_t* status) {
  const int r = blockIdx.x;
  const int b = row_seq(rm, r);
  float* dst = x + (int64_t)r * d;
  if (rm.cidx[b] > 0) {
    const float* src = state + (int64_t)(sm.base[b] + r - rm.start[b]) * d;
    for (int i = threadIdx.x; i < d; i += blockDim.x) dst[i] = src[i];
    return;
  }
  const int t = tok[r];
  const bool ok = t >= 0 && t < vocab;
  if (!ok && threadIdx.x == 0 && status) atomicOr(status, (int32_t)CAD_DEV_BAD_TOKEN);
  const T* src = table + (int64_t)(ok ? t : 0) * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) dst[i] = ok ? to_f<T>(src[i]) : 0.f;
}

hipError_t launch_loop_load(int dtype, const void* table, int vocab, int d, const int32_t* tokens, const float* state,
                            const RowMap& rm, const StateMap& sm, float* x, int32_t* status, hipStream_t s) {
  if (dtype == CAD_BF16)
    hipLaunchKernelGGL(k_loop_load<bf16_t>, dim3(rm.total), dim3(ROW_THREADS), 0, s, (const bf16_t*)table, vocab, d,
                       tokens, state, rm, sm, x, status);
  else
    hipLaunchKernelGGL(k_loop_load<float>, dim3(rm.total), dim3(ROW_THREADS), 0, s, (const float*)table, vocab, d,
                       tokens, state, rm, sm, x, status);
  return hipGetLastError();
}

// One thread per four elements of a row: the pending k-split partial sums
// are added to x in split order (their loads issued in batches of eight, so
// the row does not wait for them one by one), and the row is saved to its
// state slot.
__global__ void __launch_bounds__(ROW_THREADS) k_loop_store(float* __restrict__ x, const float* __restrict__ x_part,
                                                         int n_part, int d, float* __restrict__ state, RowMap rm,
                                                         StateMap sm) {
  const int r = blockIdx.y;
  const int i = 4 * (blockIdx.x * ROW_THREADS + threadIdx.x);
  if (i >= d) return;
  const int b = row_seq(rm, r);
  float* xr = x + (int64_t)r * d + i;
  f32x4 v = *(const f32x4*)xr;
  constexpr int PB = 8;
  for (int sp = 0; sp < n_part; sp += PB) {
    f32x4 t[PB];
#pragma unroll
    for (int j = 0; j < PB; ++j)
      t[j] = *(const f32x4*)(x_part + ((int64_t)min(sp + j, n_part - 1) * rm.total + r) * d + i);
#pragma unroll
    for (int j = 0; j < PB; ++j)
      if (sp + j < n_part) v += t[j];
  }
  if (n_part > 0) *(f32x4*)xr = v;
  // the state buffer is the caller's: plain element stores, no alignment assumed
  float* st = state + (int64_t)(sm.base[b] + r - rm.start[b]) * d + i;
#pragma unroll
  for (int e = 0; e < 4; ++e) st[e] = v[e];
}

hipError_t launch_loop_store(float* x, const float* x_part, int n_part, int d, float* state, const RowMap& rm,
                             const StateMap& sm, hipStream_t s) {
  if (n_part > 0 && !x_part) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((d / 4 + ROW_THREADS - 1) / ROW_THREADS), (unsigned)rm.total);
  hipLaunchKernelGGL(k_loop_store, grid, dim3(ROW_THREADS), 0, s, x, x_part, n_part, d, state, rm, sm);
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
  // groups past the row end hold clamped partial sums: they are neither
  // stored nor counted
#pragma unroll
  for (int j = 0; j < V4; ++j)
    if ((int)threadIdx.x + j * NT < n4)
      ss += v[j][0] * v[j][0] + v[j][1] * v[j][1] + v[j][2] * v[j][2] + v[j][3] * v[j][3];
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
  const int64_t blk = write_kv ? kv.table[(int64_t)rm.trow[b] * kv.max_blocks + pos / CAD_KV_BLOCK] : 0;
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
  T* kc = (T*)kv.k + (int64_t)rm.cidx[b] * kv.cache_stride;
  T* vc = (T*)kv.v + (int64_t)rm.cidx[b] * kv.cache_stride;
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
  // rotations: q heads then k heads (staged order), one (head, pair) per item.
  // Values past half's range (q always, k and v in the span workspace of a
  // bf16 model) are saturated there and flagged.
  constexpr bool HALF = sizeof(TQ) == 2;
  bool big = false;
  const int n_rot = (nq + nk) * half;
  for (int it = threadIdx.x; it < n_rot; it += blockDim.x) {
    const int hs = it / half, i = it % half;
    const float c = rot[i].x, s = rot[i].y;
    const float a = ld(hs * hd + i), bb = ld(hs * hd + i + half);
    const float ra = a * c - bb * s, rb = a * s + bb * c;
    if (HALF) big |= !(fabsf(ra) <= 65504.f) || !(fabsf(rb) <= 65504.f);
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
    if (HALF) big |= !(fabsf(vv) <= 65504.f);
    if (write_kv) vc[((blk * hkv + g) * hd + dd) * CAD_KV_BLOCK + slot] = from_f<T>(vv);
    if (kv.span_v) kv.span_v[((int64_t)g * hd + dd) * kv.span_cap + wrow] = f2h(vv);
  }
  if (big && status) atomicOr(status, (int32_t)CAD_DEV_F16_RANGE);
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
// Decision step after the LM head: the masked argmax of every row from the
// candidates the LM head's epilogue left (one per column tile: the tile's
// largest allowed logit and its lowest id), then the acceptance scan of every
// sequence.  A work-group of DECIDE_THREADS threads takes DECIDE_ROWS rows
// (each wave DECIDE_RB of them, every candidate load in flight at once, up
// to DECIDE_CPL per lane and chunk) and merges each row over its wave by
// lane swaps.  When one work-group covers every row it also runs the
// acceptance scan after a barrier (one thread per sequence); otherwise
// k_accept follows as a second launch.
// ---------------------------------------------------------------------------
constexpr int DECIDE_THREADS = 1024;
constexpr int DECIDE_RB = 4;    // rows per wave
constexpr int DECIDE_ROWS = DECIDE_RB * DECIDE_THREADS / 64;  // rows per work-group
constexpr int DECIDE_CPL = 4;   // candidates per lane, row and chunk

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return i >= 0 && (bi < 0 || v > bv || (v == bv && i < bi));
}

// acceptance of sequence b: COMMIT -> its rows (capped by the limit);
// VERIFY -> 1 + the leading j >= 1 with argmax[j - 1] == span[j]
__device__ __forceinline__ void accept_seq(const RowMap& rm, int b, const int32_t* span, int mode, const int32_t* limit,
                                           int lim, const int32_t* argmax, int32_t* accepted) {
  const int s0 = rm.start[b];
  int n = rm.start[b + 1] - s0;
  if (limit) n = min(n, lim);
  int acc = n;
  if (mode == CAD_VERIFY) {
    acc = 1;
    while (acc < n && argmax[s0 + acc - 1] == span[s0 + acc]) ++acc;
  }
  accepted[b] = acc;
}

template <bool ACCEPT>
__global__ void __launch_bounds__(DECIDE_THREADS) k_decide(const u32x2* __restrict__ cand, int n_cand, int rows,
                                                           RowMap rm, const int32_t* __restrict__ span, int mode,
                                                           const int32_t* limit, int32_t* __restrict__ argmax,
                                                           int32_t* __restrict__ accepted, int32_t* status) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lim = limit ? max(1, *limit) : rows;
  const int r0 = blockIdx.x * DECIDE_ROWS + wave * DECIDE_RB;
  float bv[DECIDE_RB];
  int bi[DECIDE_RB];
#pragma unroll
  for (int j = 0; j < DECIDE_RB; ++j) bv[j] = 0.f, bi[j] = -1;
  // candidate chunks in increasing column order (one chunk for up to
  // 64 * DECIDE_CPL candidates per row)
  for (int c0 = 0; c0 < n_cand && r0 < rows; c0 += 64 * DECIDE_CPL) {
    u32x2 e[DECIDE_RB][DECIDE_CPL];
#pragma unroll
    for (int j = 0; j < DECIDE_RB; ++j)
#pragma unroll
      for (int u = 0; u < DECIDE_CPL; ++u) {
        // clamped indices: every load reads a valid candidate
        const int c = min(c0 + lane + 64 * u, n_cand - 1), r = min(r0 + j, rows - 1);
        e[j][u] = cand[(int64_t)c * rows + r];
      }
#pragma unroll
    for (int j = 0; j < DECIDE_RB; ++j)
#pragma unroll
      for (int u = 0; u < DECIDE_CPL; ++u) {
        const float v = __uint_as_float(e[j][u][0]);
        const int i = (int)e[j][u][1];
        if (c0 + lane + 64 * u < n_cand && better(v, i, bv[j], bi[j])) { bv[j] = v; bi[j] = i; }
      }
  }
#pragma unroll
  for (int j = 0; j < DECIDE_RB; ++j) {
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv[j], o);
      const int oi = __shfl_xor(bi[j], o);
      if (better(ov, oi, bv[j], bi[j])) { bv[j] = ov; bi[j] = oi; }
    }
    const int r = r0 + j;
    if (lane == 0 && r < rows) {
      argmax[r] = r < lim ? bi[j] : -1;
      if (r < lim && bi[j] < 0 && status) atomicOr(status, (int32_t)CAD_DEV_EMPTY_MASK);
    }
  }
  if constexpr (ACCEPT) {
    // the barrier makes this work-group's argmax stores visible to all of it
    __syncthreads();
    if ((int)threadIdx.x < rm.n_seq) accept_seq(rm, threadIdx.x, span, mode, limit, lim, argmax, accepted);
  }
}

__global__ void k_accept(RowMap rm, const int32_t* __restrict__ span, int mode, const int32_t* limit,
                         const int32_t* __restrict__ argmax, int32_t* __restrict__ accepted) {
  const int b = threadIdx.x;
  if (b < rm.n_seq) accept_seq(rm, b, span, mode, limit, limit ? max(1, *limit) : 0, argmax, accepted);
}

hipError_t launch_decide(const uint32_t* cand, int n_cand, int rows, const RowMap& rm, const int32_t* span,
                         int mode, const int32_t* limit, int32_t* argmax, int32_t* accepted, int32_t* status,
                         hipStream_t s) {
  if (n_cand < 1 || rows < 1 || rm.n_seq > 64) return hipErrorInvalidValue;
  const int wgs = (rows + DECIDE_ROWS - 1) / DECIDE_ROWS;
  if (wgs == 1) {
    hipLaunchKernelGGL(k_decide<true>, dim3(1), dim3(DECIDE_THREADS), 0, s, (const u32x2*)cand, n_cand, rows, rm, span,
                       mode, limit, argmax, accepted, status);
  } else {
    hipLaunchKernelGGL(k_decide<false>, dim3(wgs), dim3(DECIDE_THREADS), 0, s, (const u32x2*)cand, n_cand, rows, rm,
                       span, mode, limit, argmax, accepted, status);
    hipLaunchKernelGGL(k_accept, dim3(1), dim3(64), 0, s, rm, span, mode, limit, argmax, accepted);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// suffix-match proposal (the search itself: suffix_match.h)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(SUFFIX_THREADS)
k_suffix_match(const int32_t* __restrict__ x, int64_t T, int max_n, int min_n, int K,
               int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_len,
               int64_t* __restrict__ out_pos) {
  suffix_match_body(x, T, max_n, min_n, K, out_tokens, out_len, out_pos);
}

hipError_t launch_suffix_match(const int32_t* tokens, int64_t T, int max_n, int min_n, int K,
                               int32_t* out_tokens, int32_t* out_len, int64_t* out_pos,
                               hipStream_t s) {
  hipLaunchKernelGGL(k_suffix_match, dim3(1), dim3(SUFFIX_THREADS), 0, s, tokens, T, max_n, min_n, K,
                     out_tokens, out_len, out_pos);
  return hipGetLastError();
}

// The next block's proposal straight after a readout, with no host round
// trip: the block at `pos` keeps keep = *kept rows, its prediction at the
// last kept row is the next head, written to hist[pos + keep], and the
// suffix match runs over hist[0 .. pos + keep].  out_head receives the head.
__global__ void __launch_bounds__(SUFFIX_THREADS)
k_propose_next(int32_t* __restrict__ hist, int64_t pos, const int32_t* __restrict__ kept,
               const int32_t* __restrict__ argmax, int max_n, int min_n, int K, int32_t* __restrict__ out_tokens,
               int32_t* __restrict__ out_len, int64_t* __restrict__ out_pos, int32_t* __restrict__ out_head) {
  __shared__ int32_t head;
  const int keep = *kept;
  if (threadIdx.x == 0) {
    head = argmax[keep - 1];
    hist[pos + keep] = head;
    *out_head = head;
  }
  // the barrier publishes the head (LDS) and its history store to the work-group
  __syncthreads();
  suffix_match_body(hist, pos + keep + 1, max_n, min_n, K, out_tokens, out_len, out_pos);
}

hipError_t launch_propose_next(int32_t* hist, int64_t pos, const int32_t* kept, const int32_t* argmax, int max_n,
                               int min_n, int K, int32_t* out_tokens, int32_t* out_len, int64_t* out_pos,
                               int32_t* out_head, hipStream_t s) {
  hipLaunchKernelGGL(k_propose_next, dim3(1), dim3(SUFFIX_THREADS), 0, s, hist, pos, kept, argmax, max_n, min_n, K,
                     out_tokens, out_len, out_pos, out_head);
  return hipGetLastError();
}

}  // namespace cad
