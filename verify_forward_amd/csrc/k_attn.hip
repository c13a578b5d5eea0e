// Causal span attention over the paged KV cache (GQA).
//
// Span row k of a sequence sits at absolute position L + k and attends to
// keys 0 .. L + k (the prefix cache plus the span's own keys, appended just
// before).  Query head h reads KV head h / G, G = Hq / Hkv.
//
// bf16 models (matrix cores, half operands: q arrives as half, K and V are
// widened from the bf16 cache to half while staged in LDS, P is rounded to
// half).  One work-group = one KV head x 64 query rows
// (query row = span row * G + head-in-group, so the G query heads that share
// a KV head share every K/V tile) x one partition of the key axis.  Keys are
// processed 32 at a time: the K tile [32][hd] and the V tile, stored
// token-minor in the cache ([hd][16] per block), are staged in LDS and used
// by all four waves.  Each wave owns 16 query rows and computes
//   S^T = K Q^T      (v_mfma_f32_16x16x32_f16; lane -> one query column)
//   O^T += V^T P^T   (P^T's k index is permuted to the keys the lane holds)
// so the online-softmax state of a query lives in the four lanes that hold
// its column and never needs a transpose.  Partitions write unnormalised
// partial outputs plus (max, sum) and are merged by a log-sum-exp kernel;
// with one partition the output is normalised in place.
//
// fp32 path (small reference shapes): one wave per (row, head); each lane
// runs an online softmax over a strided subset of keys, then the lanes merge.
#include "cad_internal.h"

namespace cad {

struct AttnArgs {
  const void* q;   // [rows][hq][hd]
  int rows, hq, hkv, G;
  RowMap rm;
  KVView kv;
  int32_t tstart[CAD_MAX_SEQS + 1];  // 64-row query tiles per sequence (CSR)
  int n_parts, part_len;
  float* part_o;   // [n_parts][rows * hq][hd]
  float* part_ml;  // [n_parts][rows * hq][2]
  void* out;       // [rows][hq * hd]
  int32_t* status;
  float scale_log2;  // log2(e) / sqrt(hd)
};

constexpr int AT_KEYS = 32;
constexpr int AT_PAD = 8;

template <int HD>
__global__ void __launch_bounds__(256)
k_attn_bf16(AttnArgs p) {
  constexpr int KLD = HD + AT_PAD;       // sK row stride (halves)
  constexpr int VLD = AT_KEYS + AT_PAD;  // sVt row stride (halves)
  constexpr int DS = HD / 32;            // k steps of the QK^T product
  constexpr int DB = HD / 16;            // 16-wide output blocks
  __shared__ __attribute__((aligned(16))) f16_t sK[AT_KEYS * KLD];
  __shared__ __attribute__((aligned(16))) f16_t sVt[HD * VLD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, i16 = lane & 15;
  const int kvh = blockIdx.y, part = blockIdx.z;
  // which sequence / tile
  int b = 0;
  while (b + 1 < p.rm.n_seq && p.tstart[b + 1] <= (int)blockIdx.x) ++b;
  const int tile = blockIdx.x - p.tstart[b];
  const int n_rows = p.rm.start[b + 1] - p.rm.start[b];
  const int R = n_rows * p.G;
  const int64_t L = p.rm.L[b];
  // this lane's query column
  const int qr = tile * 64 + wave * 16 + i16;
  const bool q_ok = qr < R;
  const int k_local = q_ok ? qr / p.G : 0;
  const int head = kvh * p.G + (q_ok ? qr % p.G : 0);
  const int grow = p.rm.start[b] + k_local;
  const int64_t q_last_key = L + k_local;  // inclusive causal limit
  // work-group key range
  const int last_row = min((tile * 64 + 63) / p.G, n_rows - 1);
  const int64_t wg_keys_end = L + last_row + 1;
  const int64_t k_begin = (int64_t)part * p.part_len;
  const int64_t k_end = min((int64_t)(part + 1) * p.part_len, wg_keys_end);

  // Q fragments (operand B of S^T = K Q^T): Q[query][ds*32 + 8*g4 .. +7]
  u32x4 qf[DS];
  const f16_t* qsrc = (const f16_t*)p.q + ((int64_t)grow * p.hq + head) * HD;
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    qf[ds] = q_ok ? *(const u32x4*)(qsrc + ds * 32 + g4 * 8) : u32x4{0u, 0u, 0u, 0u};
  }
  f32x4 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const bf16_t* kbase = (const bf16_t*)p.kv.k;
  const bf16_t* vbase = (const bf16_t*)p.kv.v;
  const int32_t* table = p.kv.table + (int64_t)b * p.kv.max_blocks;

  for (int64_t kt = k_begin; kt < k_end; kt += AT_KEYS) {
    // ---- stage K [32][HD] and V^T [HD][32] in LDS ----
    constexpr int KCH = AT_KEYS * HD / 8;  // 16-byte chunks of the K tile
    for (int c = tid; c < KCH; c += 256) {
      const int key = c / (HD / 8), c8 = c % (HD / 8);
      const int64_t kk = kt + key;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (kk < k_end) {
        const int64_t blk = table[kk / CAD_KV_BLOCK];
        if (blk >= 0 && blk < p.kv.num_blocks)
          v = bf16x8_to_f16x8(
              *(const u32x4*)(kbase + ((blk * p.hkv + kvh) * CAD_KV_BLOCK + kk % CAD_KV_BLOCK) * HD + c8 * 8));
        else if (p.status)
          atomicOr(p.status, (int32_t)CAD_DEV_BAD_BLOCK);
      }
      *(u32x4*)(&sK[key * KLD + c8 * 8]) = v;
    }
    constexpr int VCH = 2 * HD * 2;  // 2 blocks x HD rows x 2 chunks of 8 tokens
    for (int c = tid; c < VCH; c += 256) {
      const int half = c & 1, d = (c >> 1) % HD, kb = (c >> 1) / HD;
      const int64_t k0 = kt + kb * 16 + half * 8;  // first token of the chunk
      u32x4 v = {0u, 0u, 0u, 0u};
      if (k0 < k_end) {
        const int64_t blk = table[k0 / CAD_KV_BLOCK];
        if (blk >= 0 && blk < p.kv.num_blocks) {
          v = bf16x8_to_f16x8(*(const u32x4*)(vbase + ((blk * p.hkv + kvh) * HD + d) * CAD_KV_BLOCK + half * 8));
          // zero tokens of the chunk that lie past the range end
          const int64_t valid = k_end - k0;
          if (valid < 8) {
            uint16_t* e = (uint16_t*)&v;
            for (int j = (int)valid; j < 8; ++j) e[j] = 0;
          }
        }
      }
      *(u32x4*)(&sVt[d * VLD + kb * 16 + half * 8]) = v;
    }
    __syncthreads();

    // ---- S^T for the two 16-key blocks ----
    f32x4 s[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      s[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const u32x4 kf = *(const u32x4*)(&sK[(i * 16 + i16) * KLD + ds * 32 + g4 * 8]);
        s[i] = mfma16(kf, qf[ds], s[i]);
      }
    }
    // lane holds S[query i16][key kt + 16 i + 4 g4 + r]
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t key = kt + i * 16 + g4 * 4 + r;
        const bool ok = q_ok && key < k_end && key <= q_last_key;
        const float v = ok ? s[i][r] * p.scale_log2 : -INFINITY;
        s[i][r] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    float alpha = 1.f;
    u32x2 pk[2];
    if (m_new == -INFINITY) {
      pk[0] = u32x2{0u, 0u};
      pk[1] = u32x2{0u, 0u};
    } else {
      alpha = exp2f(m_run - m_new);
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[r] = exp2f(s[i][r] - m_new);
          psum += e[r];
        }
        pk[i] = u32x2{__builtin_bit_cast(uint32_t, f16x2{(f16_t)e[0], (f16_t)e[1]}),
                      __builtin_bit_cast(uint32_t, f16x2{(f16_t)e[2], (f16_t)e[3]})};
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
    }
    const u32x4 pf = {pk[0][0], pk[0][1], pk[1][0], pk[1][1]};
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      const f16_t* vr = &sVt[(d * 16 + i16) * VLD];
      const u32x2 v0 = *(const u32x2*)(vr + g4 * 4);
      const u32x2 v1 = *(const u32x2*)(vr + 16 + g4 * 4);
      const u32x4 vf = {v0[0], v0[1], v1[0], v1[1]};
      o[d] *= alpha;
      o[d] = mfma16(vf, pf, o[d]);
    }
    __syncthreads();
  }
  // combine the four lanes of each query column
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (!q_ok) return;
  // lane holds O^T[d = 16 db + 4 g4 + r][query i16]
  if (p.n_parts == 1) {
    f16_t* out = (f16_t*)p.out + ((int64_t)grow * p.hq + head) * HD;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      const int dd = d * 16 + g4 * 4;
      const uint32_t lo = __builtin_bit_cast(uint32_t, f16x2{f2h(o[d][0] * inv), f2h(o[d][1] * inv)});
      const uint32_t hi = __builtin_bit_cast(uint32_t, f16x2{f2h(o[d][2] * inv), f2h(o[d][3] * inv)});
      *(u32x2*)(out + dd) = u32x2{lo, hi};
    }
  } else {
    const int64_t qi = (int64_t)part * p.rows * p.hq + (int64_t)grow * p.hq + head;
    float* po = p.part_o + qi * HD;
#pragma unroll
    for (int d = 0; d < DB; ++d) *(f32x4*)(po + d * 16 + g4 * 4) = o[d];
    if (g4 == 0) {
      p.part_ml[qi * 2 + 0] = m_run;
      p.part_ml[qi * 2 + 1] = l_run;
    }
  }
}

// log-sum-exp merge of the partitions (base-2 exponent, as produced above)
template <typename T>
__global__ void k_attn_merge(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                             int n_parts, int64_t nq, int hd, T* __restrict__ out) {
  const int64_t qi = blockIdx.x;
  float m = -INFINITY;
  for (int pp = 0; pp < n_parts; ++pp) {
    const float l = part_ml[((int64_t)pp * nq + qi) * 2 + 1];
    if (l > 0.f) m = fmaxf(m, part_ml[((int64_t)pp * nq + qi) * 2]);
  }
  for (int d = threadIdx.x; d < hd; d += blockDim.x) {
    float num = 0.f, den = 0.f;
    for (int pp = 0; pp < n_parts; ++pp) {
      const float l = part_ml[((int64_t)pp * nq + qi) * 2 + 1];
      if (!(l > 0.f)) continue;
      const float w = exp2f(part_ml[((int64_t)pp * nq + qi) * 2] - m);
      num += w * part_o[((int64_t)pp * nq + qi) * hd + d];
      den += w * l;
    }
    out[qi * hd + d] = from_f<T>(den > 0.f ? num / den : 0.f);
  }
}

// ---------------------------------------------------------------------------
// fp32 path
// ---------------------------------------------------------------------------
constexpr int F32_MAX_HD = 128;

__global__ void __launch_bounds__(64)
k_attn_f32(AttnArgs p, int hd) {
  __shared__ float sq[F32_MAX_HD];
  const int r = blockIdx.x, head = blockIdx.y, lane = threadIdx.x;
  const int b = row_seq(p.rm, r);
  const int64_t pos = p.rm.L[b] + (r - p.rm.start[b]);
  const int g = head / p.G;
  const float* q = (const float*)p.q + ((int64_t)r * p.hq + head) * hd;
  for (int d = lane; d < hd; d += 64) sq[d] = q[d];
  __syncthreads();
  const float* kc = (const float*)p.kv.k;
  const float* vc = (const float*)p.kv.v;
  const int32_t* table = p.kv.table + (int64_t)b * p.kv.max_blocks;
  const float scale = 1.0f / sqrtf((float)hd);
  float m = -INFINITY, l = 0.f;
  float o[F32_MAX_HD];
  for (int d = 0; d < hd; ++d) o[d] = 0.f;
  for (int64_t j = lane; j <= pos; j += 64) {
    const int64_t blk = table[j / CAD_KV_BLOCK];
    if (blk < 0 || blk >= p.kv.num_blocks) {
      if (p.status) atomicOr(p.status, (int32_t)CAD_DEV_BAD_BLOCK);
      continue;
    }
    const int slot = (int)(j % CAD_KV_BLOCK);
    const float* kr = kc + ((blk * p.hkv + g) * CAD_KV_BLOCK + slot) * hd;
    float s = 0.f;
    for (int d = 0; d < hd; ++d) s += sq[d] * kr[d];
    s *= scale;
    const float m_new = fmaxf(m, s);
    const float a = __expf(m - m_new), e = __expf(s - m_new);
    l = l * a + e;
    const float* vr = vc + ((blk * p.hkv + g) * hd) * CAD_KV_BLOCK + slot;
    for (int d = 0; d < hd; ++d) o[d] = o[d] * a + e * vr[(int64_t)d * CAD_KV_BLOCK];
    m = m_new;
  }
  float mw = m;
  for (int off = 32; off > 0; off >>= 1) mw = fmaxf(mw, __shfl_xor(mw, off));
  const float w = (m == -INFINITY) ? 0.f : __expf(m - mw);
  float lt = l * w;
  for (int off = 32; off > 0; off >>= 1) lt += __shfl_xor(lt, off);
  float* out = (float*)p.out + ((int64_t)r * p.hq + head) * hd;
  for (int d = 0; d < hd; ++d) {
    float v = o[d] * w;
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) out[d] = v / lt;
  }
}

int attention_parts(int rows, int hq, int hkv, int64_t max_keys, int* part_len) {
  const int G = hq / hkv;
  const int tiles = (rows * G + 63) / 64;
  const int base = hkv * tiles;
  int parts = (512 + base - 1) / base;
  const int64_t min_len = 256;
  const int64_t cap = (max_keys + min_len - 1) / min_len;
  if (parts > cap) parts = (int)cap;
  if (parts < 1) parts = 1;
  int64_t len = (max_keys + parts - 1) / parts;
  len = (len + AT_KEYS - 1) / AT_KEYS * AT_KEYS;
  *part_len = (int)len;
  return (int)((max_keys + len - 1) / len);
}

hipError_t launch_attention(int dtype, const void* q, int rows, int hq, int hkv, int hd,
                            const RowMap& rm, KVView kv, int n_parts, int part_len,
                            float* part_o, float* part_ml, void* out, int32_t* status,
                            hipStream_t s) {
  AttnArgs a;
  a.q = q;
  a.rows = rows;
  a.hq = hq;
  a.hkv = hkv;
  a.G = hq / hkv;
  a.rm = rm;
  a.kv = kv;
  a.n_parts = n_parts;
  a.part_len = part_len;
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.out = out;
  a.status = status;
  a.scale_log2 = 1.4426950408889634f / sqrtf((float)hd);
  if (dtype == CAD_F32) {
    hipLaunchKernelGGL(k_attn_f32, dim3(rows, hq), dim3(64), 0, s, a, hd);
    return hipGetLastError();
  }
  int nt = 0;
  a.tstart[0] = 0;
  for (int b = 0; b < rm.n_seq; ++b) {
    const int R = (rm.start[b + 1] - rm.start[b]) * a.G;
    nt += (R + 63) / 64;
    a.tstart[b + 1] = nt;
  }
  dim3 grid(nt, hkv, n_parts);
  if (hd == 64)
    hipLaunchKernelGGL(k_attn_bf16<64>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_attn_bf16<128>, grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_parts == 1) return e;
  const int64_t nq = (int64_t)rows * hq;
  hipLaunchKernelGGL(k_attn_merge<f16_t>, dim3((unsigned)nq), dim3(hd), 0, s, part_o, part_ml,
                     n_parts, nq, hd, (f16_t*)out);
  return hipGetLastError();
}

}  // namespace cad
