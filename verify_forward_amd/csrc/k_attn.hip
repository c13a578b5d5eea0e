// Causal span attention over the paged KV cache (GQA).
//
// Span row k of a sequence sits at absolute position L + k and attends to
// keys 0 .. L + k (the prefix cache plus the span's own keys, appended just
// before).  Query head h reads KV head h / G, G = Hq / Hkv.
//
// bf16 models (matrix cores, half operands: q arrives as half, K and V are
// widened from the bf16 cache to half while staged in LDS, P is rounded to
// half).  One work-group = one KV head x 256 query rows (128 for calls with
// at most 128 query rows; query row = span row * G + head-in-group, so the G
// query heads that share a KV head share every K/V tile) x one partition of
// the key axis.  Keys are processed 64 at a
// time through a double-buffered LDS stage: the K tile [64][hd] and the V
// tile, stored token-minor in the cache ([hd][16] per block) and kept
// transposed in LDS, are loaded once per work-group and read by all its
// waves; the global loads of tile t+1 are in flight while tile t is on the
// matrix cores.  Each wave owns 32 query rows (two 16-column blocks) and
// computes
//   S^T = K Q^T      (v_mfma_f32_16x16x32_f16; lane -> one query column)
//   O^T += V^T P^T   (the key order inside each 32-key group of the LDS V
//                     tile is permuted so that the eight keys a lane feeds as
//                     P^T are exactly the eight it holds in S^T)
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
  const void* q;     // [rows][hq][hd]: fp32 (fp32 models) or the half hi plane
  const void* q_lo;  // bf16 models: the half remainder plane
  int rows, hq, hkv, G;
  RowMap rm;
  KVView kv;
  int32_t tstart[CAD_MAX_SEQS + 1];  // query tiles per sequence (CSR)
  int n_parts;
  float* part_o;   // [n_parts][rows * hq][hd]
  float* part_ml;  // [n_parts][rows * hq][2]
  void* out;       // [rows][hq * hd]: fp32 (fp32 models) or the bf16 hi plane (bf16 models)
  void* out_lo;    // bf16 models: the bf16 lo plane
  int32_t* status;
  float scale_log2;  // log2(e) / sqrt(hd)
  float pos_inf;     // +inf
};

constexpr int FA_KT = 64;                  // keys per tile
// Work-group shapes: eight waves of 32 query rows (two waves per SIMD) for
// long spans; four waves of 16 rows (several work-groups per CU, twice the
// work-groups over the key axis to spread the cache stream wider) when the
// call's sequences average at most 64 query rows (short spans, and batched
// serving, where most sequences take a one-token step).  (One wave per SIMD with 48 or 64 rows
// each, which reads each K/V fragment from LDS once for more queries,
// measured 2.6x slower: nothing hides LDS and softmax latency then.)
inline int attn_qt(int query_rows, int n_seq) { return query_rows <= 64 * n_seq ? 64 : 256; }

// Work-group -> (query tile, KV head, key partition).  The query tiles that
// read the same KV head and key range are placed on one XCD (work-group ids
// are dealt to the eight XCDs round-robin) so that their shared K/V tiles
// are fetched from HBM once and then hit that XCD's L2.
__device__ __forceinline__ void attn_tile_of(int& x, int& y, int& z) {
  const int X = gridDim.x, Y = gridDim.y, Z = gridDim.z;
  const int id = blockIdx.x + X * (blockIdx.y + Y * blockIdx.z);
  if ((Y * Z) % 8 != 0) {
    x = blockIdx.x; y = blockIdx.y; z = blockIdx.z;
    return;
  }
  const int xcd = id & 7, slot = id >> 3;
  const int gi = xcd + 8 * (slot / X);
  x = slot % X;
  y = gi % Y;
  z = gi / Y;
}

// Online softmax keeps a per-query running maximum in exp2 units and moves
// it only when a tile raises some query's maximum by more than this margin,
// so the O rescale is skipped on most tiles; until then the unnormalised
// weights stay below 2^FA_LAZY, far inside half's range.
constexpr float FA_LAZY = 8.0f;

// max(a, b) as the median of (a, b, +inf): one instruction, where fmaxf first
// quiets each operand that comes straight from the matrix cores or a lane
// swap (no NaN can reach the scores: masked keys are -inf, every product is
// finite).  `inf` arrives as a kernel argument so that the compiler does not
// turn the median back into fmaxf.
__device__ __forceinline__ float max_raw(float a, float b, float inf) { return __builtin_amdgcn_fmed3f(a, b, inf); }

// max over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the four row groups of a
// wave that hold one query column), by the two half-swapping lane
// permutations instead of LDS-routed shuffles
__device__ __forceinline__ float max_col4(float m, float inf) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  m = max_raw(__uint_as_float(a[0]), __uint_as_float(a[1]), inf);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return max_raw(__uint_as_float(b[0]), __uint_as_float(b[1]), inf);
}

template <int HD, int NW, int QB>
__global__ void __launch_bounds__(64 * NW, 8 / NW)
k_attn_bf16(AttnArgs p) {
  constexpr int FA_NT = 64 * NW;            // threads per work-group
  constexpr int QPW = 16 * QB;              // query rows per wave (QB 16-column blocks)
  constexpr int FA_QT = QPW * NW;           // query rows per work-group
  // LDS row strides (halves) with 32 bytes of padding (measured 2 % faster
  // than 16 bytes for the eight-wave shape)
  constexpr int KLD = HD + 16;         // sK
  constexpr int VLD = FA_KT + 16;      // sV
  constexpr int DS = HD / 32;          // k steps of S^T = K Q^T
  constexpr int DB = HD / 16;          // 16-row d blocks of O^T
  constexpr int TBLK = FA_KT / CAD_KV_BLOCK;   // cache blocks per tile
  constexpr int TPB = FA_NT / TBLK;            // staging threads per cache block
  constexpr int KCH = CAD_KV_BLOCK * HD / 8 / TPB;  // 16-byte K chunks per thread and tile
  constexpr int VCH = HD * CAD_KV_BLOCK / 8 / TPB;  // 16-byte V chunks per thread and tile
  static_assert(KCH >= 1 && KCH * TPB * 8 == CAD_KV_BLOCK * HD && VCH * TPB * 8 == HD * CAD_KV_BLOCK,
                "tile split");
  static_assert(TPB % 64 == 0, "a wave stages from one cache block");
  __shared__ __attribute__((aligned(16))) f16_t sK[2][FA_KT * KLD];
  __shared__ __attribute__((aligned(16))) f16_t sV[2][HD * VLD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, i16 = lane & 15;
  int bx, kvh, part;
  attn_tile_of(bx, kvh, part);
  int b = 0;
  while (b + 1 < p.rm.n_seq && p.tstart[b + 1] <= bx) ++b;
  const int tile = bx - p.tstart[b];
  const int n_rows = p.rm.start[b + 1] - p.rm.start[b];
  const int R = n_rows * p.G;
  const int64_t L = p.rm.L[b];
  const int q_first = tile * FA_QT;
  const int q_wave = q_first + wave * QPW;
  const bool wave_active = q_wave < R;
  // Keys of this work-group.  The key axis of a query tile is the cached
  // keys 0 .. L - 1 (paged bf16 cache, TA tiles of 64 keys, the last one
  // possibly short) followed by this call's own keys L .. causal_end - 1
  // (half-precision span workspace, TB tiles).  The n_parts partitions take
  // equal runs of these TA + TB tiles (to one tile); a partition's cached
  // tiles are its segment A and its span tiles its segment B, each read from
  // its own source.
  const int q_last = min(q_first + FA_QT, R) - 1;
  const int64_t causal_end = L + q_last / p.G + 1;
  const int64_t TA = (L + FA_KT - 1) / FA_KT, TB = (causal_end - L + FA_KT - 1) / FA_KT;
  const int64_t t0 = (TA + TB) * part / p.n_parts, t1 = (TA + TB) * (part + 1) / p.n_parts;
  const int64_t a_begin = min(t0, TA) * FA_KT;
  const int64_t a_end = min(min(t1, TA) * FA_KT, L);
  const int64_t b_begin = L + max(t0 - TA, (int64_t)0) * FA_KT;
  const int64_t b_end = min(L + max(t1 - TA, (int64_t)0) * FA_KT, causal_end);
  const int nA = (int)(min(t1, TA) - min(t0, TA));
  const int n_tiles = (int)(t1 - t0);
  auto tile_start = [&](int t) -> int64_t {
    return t < nA ? a_begin + (int64_t)t * FA_KT : b_begin + (int64_t)(t - nA) * FA_KT;
  };
  auto tile_end = [&](int t) -> int64_t { return t < nA ? a_end : b_end; };
  // causal limit shared by every query of the wave (its first query's)
  const int64_t wave_min_last = L + q_wave / p.G;

  // this lane's query columns.  q arrives as two half planes (hi, and the
  // half-rounded remainder lo); S^T takes two products per K fragment, so q
  // enters the scores with ~22 significant bits.  The hi fragments stay in
  // registers; the lo fragments too with one query block per wave, and in
  // LDS (read only by this wave) with two.
  constexpr bool QLO_LDS = QB >= 2;
  constexpr int QLD = HD + 16;  // sQlo row stride (halves)
  __shared__ __attribute__((aligned(16))) f16_t sQlo[QLO_LDS ? NW * QPW * QLD : 8];
  bool q_ok[QB];
  int64_t q_last_key[QB];  // this lane's last visible key
  int64_t qrow[QB];
  u32x4 qf[QB][DS], qfl[QLO_LDS ? 1 : QB][DS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = q_wave + qb * 16 + i16;
    q_ok[qb] = qi < R;
    const int k_local = q_ok[qb] ? qi / p.G : 0;
    const int head = kvh * p.G + (q_ok[qb] ? qi % p.G : 0);
    q_last_key[qb] = L + k_local;
    qrow[qb] = (int64_t)(p.rm.start[b] + k_local) * p.hq + head;  // index of (row, head)
    const f16_t* qsrc = (const f16_t*)p.q + qrow[qb] * HD;
    const f16_t* qlsrc = (const f16_t*)p.q_lo + qrow[qb] * HD;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const u32x4 zero = {0u, 0u, 0u, 0u};
      qf[qb][ds] = q_ok[qb] ? *(const u32x4*)(qsrc + ds * 32 + g4 * 8) : zero;
      const u32x4 vl = q_ok[qb] ? *(const u32x4*)(qlsrc + ds * 32 + g4 * 8) : zero;
      if (QLO_LDS)
        *(u32x4*)(&sQlo[(wave * QPW + qb * 16 + i16) * QLD + ds * 32 + g4 * 8]) = vl;
      else
        qfl[QLO_LDS ? 0 : qb][ds] = vl;
    }
  }
  f32x4 o[DB][QB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) o[d][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // finite start: exp2 of (masked score - m_run) is 0, never NaN
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) m_run[qb] = -1e30f, l_run[qb] = 0.f;

  const int32_t* table = p.kv.table + (int64_t)p.rm.trow[b] * p.kv.max_blocks;
  // Staging: the threads of wave w copy cache block jb = w / (TPB / 64) of
  // each tile, so the block id is uniform over the wave (a scalar load).
  const int jb = __builtin_amdgcn_readfirstlane(tid / TPB);
  const int ct = tid % TPB;
  const int64_t kv_blk_stride = (int64_t)p.hkv * CAD_KV_BLOCK * HD;  // elements per cache block
  const int64_t coff = (int64_t)p.rm.cidx[b] * p.kv.cache_stride + (int64_t)kvh * CAD_KV_BLOCK * HD;
  const bf16_t* kbase = (const bf16_t*)p.kv.k + coff;
  const bf16_t* vbase = (const bf16_t*)p.kv.v + coff;
  // cache block of tile t for this wave (lane 0 of the result), or -1 when
  // the tile's part of the key range does not reach it (then nothing is
  // read); unused by span tiles.  Lanes 32..63 read the next block's id
  // (clamped to the range): the value is then not wave-uniform, stays in a
  // vector register, and the wait for it falls where lane 0 is read a tile
  // later instead of right after the load.
  // The load is unconditional (index clamped into the range, entry 0 for
  // span tiles or an empty range) so that no path overwrites its register
  // while it is in flight; block_used says whether the tile reads the block.
  const int blast = a_end > a_begin ? (int)((a_end - 1) / CAD_KV_BLOCK) : 0;
  auto block_used = [&](int t) -> bool {
    return t < nA && a_begin + (int64_t)t * FA_KT + jb * CAD_KV_BLOCK < a_end;
  };
  auto block_of = [&](int t) -> int32_t {
    const int64_t first_key = a_begin + (int64_t)t * FA_KT + jb * CAD_KV_BLOCK;
    const int bi = t < nA ? min((int)(first_key / CAD_KV_BLOCK), blast) : 0;
    return table[min(bi + (lane >> 5), blast)];
  };
  // span workspace rows of this sequence: row pstart + (key - L)
  const int64_t span_row0 = p.rm.pstart[b];
  const f16_t* span_k = p.kv.span_k;
  const f16_t* span_v = p.kv.span_v;
  u32x4 rk[KCH], rv[VCH];
  int nvalid_pend = 0;  // valid keys of this wave's cache block in the staged tile
  bool span_pend = false;  // the staged tile comes from the span workspace
  // Every load below reads valid memory (a clamped block, or the sequence's
  // 64-row padded workspace region) and is unconditional; out-of-range keys
  // are zeroed afterwards, so the waits for tile t + 1 never cover extra work.
  auto gload = [&](int t, int32_t blkv, bool used) {
    const bool span_tile = t >= nA;  // wave-uniform
    const int64_t bb = used ? __builtin_amdgcn_readlane(blkv, 0) : -1;
    const int64_t k0 = tile_start(t) + jb * CAD_KV_BLOCK;  // first key of this wave's block
    const bool ok = span_tile || (bb >= 0 && bb < p.kv.num_blocks);
    if (!span_tile && bb >= 0 && !ok && p.status && ct == 0) atomicOr(p.status, (int32_t)CAD_DEV_BAD_BLOCK);
    span_pend = span_tile;
    const int64_t rem = tile_end(t) - k0;  // keys left in the segment from k0 (clamped in 32-bit below)
    nvalid_pend = !ok ? 0 : rem >= CAD_KV_BLOCK ? CAD_KV_BLOCK : rem > 0 ? (int)rem : 0;
    const bf16_t* kb = kbase + (ok && !span_tile ? bb : 0) * kv_blk_stride;
    const bf16_t* vb = vbase + (ok && !span_tile ? bb : 0) * kv_blk_stride;
    const int64_t srow = span_row0 + (k0 - L);  // span workspace row of key k0
    // raw loads only: the registers are not touched again until sstore, so
    // the wait for them lands at the end of the tile, not right here
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = ct + TPB * i;  // [16 keys][HD / 8 chunks]
      const int key = c / (HD / 8), c8 = c % (HD / 8);
      const u32x4* src = span_tile ? (const u32x4*)(span_k + ((srow + key) * p.hkv + kvh) * HD + c8 * 8)
                                   : (const u32x4*)(kb + c * 8);
      rk[i] = *src;
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = ct + TPB * i;  // [HD rows][2 chunks of 8 tokens]
      const int d = c >> 1, hf = c & 1;
      const u32x4* src = span_tile
                             ? (const u32x4*)(span_v + ((int64_t)kvh * HD + d) * p.kv.span_cap + srow + 8 * hf)
                             : (const u32x4*)(vb + c * 8);
      rv[i] = *src;
    }
  };
  auto sstore = [&](int buf) {
    // keys past the range are zeroed here (stale slots may hold anything);
    // nvalid_pend is wave-uniform and below a full block only at the ends
    // of the key range
    if (nvalid_pend < CAD_KV_BLOCK) {
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int kin = (ct + TPB * i) / (HD / 8);
        if (kin >= nvalid_pend) rk[i] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < VCH; ++i) {
        const int nv = nvalid_pend - 8 * ((ct + TPB * i) & 1);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t keep = (2 * w + 1 < nv) ? 0xFFFFFFFFu : (2 * w < nv ? 0x0000FFFFu : 0u);
          rv[i][w] &= keep;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = ct + TPB * i;
      const int kin = c / (HD / 8), c8 = c % (HD / 8);
      const int key = jb * CAD_KV_BLOCK + kin;
      *(u32x4*)(&sK[buf][key * KLD + c8 * 8]) = span_pend ? rk[i] : bf16x8_to_f16x8(rk[i]);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = ct + TPB * i;
      const int d = c >> 1, hf = c & 1;
      // tile keys 16 jb + 8 hf + e (e < 8).  Inside its 32-key group (32 ks
      // + 16 (jb & 1) + 8 hf + e) key 16 h + 4 j + r sits at column 8 j + 4 h
      // + r: the eight columns 8 j .. 8 j + 7 then hold keys 4 j .. 4 j + 3
      // and 16 + 4 j .. 16 + 4 j + 3, the keys lane group j holds in S^T.
      const u32x4 h = span_pend ? rv[i] : bf16x8_to_f16x8(rv[i]);
      const int col = (jb >> 1) * 32 + 16 * hf + 4 * (jb & 1);
      f16_t* row = &sV[buf][d * VLD + col];
      *(u32x2*)(row) = u32x2{h[0], h[1]};      // e = 0..3 -> j = 2 hf
      *(u32x2*)(row + 8) = u32x2{h[2], h[3]};  // e = 4..7 -> j = 2 hf + 1
    }
  };

  // Tile t + 1 is loaded into registers while tile t is on the matrix cores
  // and written to the other LDS buffer at the end of the iteration (that
  // buffer was last read before the barrier that closed tile t - 1).  Block
  // ids run one more tile ahead.
  int32_t blk = block_of(0);
  if (n_tiles > 0) {
    gload(0, blk, block_used(0));
    sstore(0);
  }
  blk = block_of(1);
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const int64_t kt = tile_start(t);
    const bool more = t + 1 < n_tiles;
    if (more) gload(t + 1, blk, block_used(t + 1));
    const int32_t blk_next = block_of(t + 2);
    if (wave_active) {
      // ---- S^T = K Q^T for four 16-key blocks x two 16-query blocks ----
      f32x4 s[4][QB];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        u32x4 ql[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          ql[qb] = QLO_LDS ? *(const u32x4*)(&sQlo[(wave * QPW + qb * 16 + i16) * QLD + ds * 32 + g4 * 8])
                           : qfl[QLO_LDS ? 0 : qb][ds];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const u32x4 kf = *(const u32x4*)(&sK[buf][(kb * 16 + i16) * KLD + ds * 32 + g4 * 8]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            s[kb][qb] = mfma16(kf, qf[qb][ds], s[kb][qb]);
            s[kb][qb] = mfma16(kf, ql[qb], s[kb][qb]);
          }
        }
      }
      // lane holds S[query (qb, i16)][key kt + 16 kb + 4 g4 + r]
      const int end_rel = (int)min<int64_t>(tile_end(t) - kt, FA_KT);
      const bool need_mask = kt + FA_KT - 1 > wave_min_last || end_rel < FA_KT;
      float mx[QB];
      bool grow = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (need_mask) {
          const int lim = (int)max<int64_t>(min<int64_t>(q_last_key[qb] - kt + 1, end_rel), 0);
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (kb * 16 + g4 * 4 + r >= lim) s[kb][qb][r] = -INFINITY;
        }
        float mk[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          mk[kb] = fmaxf(max_raw(s[kb][qb][0], s[kb][qb][1], p.pos_inf), max_raw(s[kb][qb][2], s[kb][qb][3], p.pos_inf));
        const float m = max_col4(fmaxf(fmaxf(mk[0], mk[1]), fmaxf(mk[2], mk[3])), p.pos_inf);
        mx[qb] = m * p.scale_log2;
        grow |= mx[qb] > m_run[qb] + FA_LAZY;
      }
      if (__ballot(grow)) {  // some query's maximum moved: rescale (wave-uniform branch)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float m_new = fmaxf(m_run[qb], mx[qb]);
          const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
          m_run[qb] = m_new;
          l_run[qb] *= alpha;
#pragma unroll
          for (int d = 0; d < DB; ++d) o[d][qb] *= alpha;
        }
      }
      u32x4 pf[QB][2];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float nm = -m_run[qb];
        // the row sum takes the weights as rounded for the matrix cores
        // (pairs summed by a half dot product with (1, 1) into fp32), so the
        // numerator and the denominator see the same P
        float psum = 0.f;
        const f16x2 ones = {(f16_t)1.0f, (f16_t)1.0f};
        uint32_t pk[8];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          float e[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][r], p.scale_log2, nm));
          // round to nearest (unbiased), weights are in [0, 2^FA_LAZY]
          const f16x2 e01 = {(f16_t)e[0], (f16_t)e[1]};
          const f16x2 e23 = {(f16_t)e[2], (f16_t)e[3]};
          psum = __builtin_amdgcn_fdot2(e01, ones, psum, false);
          psum = __builtin_amdgcn_fdot2(e23, ones, psum, false);
          pk[kb * 2 + 0] = __builtin_bit_cast(uint32_t, e01);
          pk[kb * 2 + 1] = __builtin_bit_cast(uint32_t, e23);
        }
        l_run[qb] += psum;
        // k step ks covers key blocks 2 ks and 2 ks + 1
        pf[qb][0] = u32x4{pk[0], pk[1], pk[2], pk[3]};
        pf[qb][1] = u32x4{pk[4], pk[5], pk[6], pk[7]};
      }
      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          const u32x4 vf = *(const u32x4*)(&sV[buf][(d * 16 + i16) * VLD + ks * 32 + g4 * 8]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[d][qb] = mfma16(vf, pf[qb][ks], o[d][qb]);
        }
    }
    if (more) sstore(buf ^ 1);
    blk = blk_next;
    __syncthreads();
  }
  if (!wave_active) return;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    // combine the four lanes of each query column
    float l = l_run[qb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (!q_ok[qb]) continue;
    // lane holds O^T[d = 16 db + 4 g4 + r][query]
    if (p.n_parts == 1) {
      bf16_t* out = (bf16_t*)p.out + qrow[qb] * HD;
      bf16_t* out_lo = (bf16_t*)p.out_lo + qrow[qb] * HD;
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        bf16_t hi[4], lo[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) split_bf16(o[d][qb][r] * inv, hi[r], lo[r]);
        const int dd = d * 16 + g4 * 4;
        *(u32x2*)(out + dd) = u32x2{hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16)};
        *(u32x2*)(out_lo + dd) = u32x2{lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16)};
      }
    } else {
      // partial: unnormalised O, and (m, l) with m in exp2 units; a query
      // that saw no key in this partition has l = 0 and is skipped by the merge
      const int64_t qi = (int64_t)part * p.rows * p.hq + qrow[qb];
      float* po = p.part_o + qi * HD;
#pragma unroll
      for (int d = 0; d < DB; ++d) *(f32x4*)(po + d * 16 + g4 * 4) = o[d][qb];
      if (g4 == 0) {
        p.part_ml[qi * 2 + 0] = m_run[qb];
        p.part_ml[qi * 2 + 1] = l;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Short spans: every sequence of the call has at most 16 query rows per KV
// head (N <= 16 / G).  One work-group = one (sequence, KV head, key
// partition); its four waves take the partition's 32-key tiles in turn, each
// with its own online softmax over the same query columns (one 16-column
// block), and K and V go from the paged cache (or the span workspace)
// straight into matrix-core fragments: no LDS stage and no barrier until
// the four waves combine their states at the end.  Every wave computes (the
// LDS-staged kernel gives such a call one computing wave per work-group),
// and each keeps one tile in flight while it works on the previous one.
//   S^T = K (Q_hi + Q_lo)^T: lane (g, i) supplies key 16 kb + i, dims
//     32 ds + 8 g .. + 7; it then holds keys 16 kb + 4 g + r of query i.
//   O^T += V^T P^T: as its k index 8 g + e the V fragment takes key 4 g + e
//     of the tile's first block (e < 4) and key 4 g + e - 4 of its second,
//     exactly the keys lane (g, i) holds in S^T, so P^T is formed in place.
// Cached K and V are widened from bf16 to half exactly; the span's own keys
// come from the half-precision span workspace.  Partials use the layout of
// the LDS-staged kernel, so the same merge follows.
// ---------------------------------------------------------------------------
constexpr int DEC_KT = 32;  // keys per tile: two cache blocks

template <int HD>
__global__ void __launch_bounds__(256, 2) k_attn_dec(AttnArgs p) {
  constexpr int DS = HD / 32, DB = HD / 16;
  // wave index made provably uniform, so that tile, block and base-pointer
  // arithmetic stays scalar and each load needs one 32-bit lane offset
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, i16 = lane & 15;
  const int part = blockIdx.x % p.n_parts;
  const int bh = blockIdx.x / p.n_parts;
  const int kvh = bh % p.hkv, b = bh / p.hkv;
  const int n_rows = p.rm.start[b + 1] - p.rm.start[b];
  const int R = n_rows * p.G;  // <= 16 (checked by the launcher)
  const int64_t L = p.rm.L[b];
  // this lane's query column
  const bool q_ok = i16 < R;
  const int k_local = q_ok ? i16 / p.G : 0;
  // key axis: TA cached tiles (keys 0 .. L - 1, the last possibly short) and
  // one span tile (keys L .. L + n_rows - 1, n_rows <= 16); the partitions
  // take equal runs of these tiles, the waves every fourth tile of a run
  const int64_t TA = (L + DEC_KT - 1) / DEC_KT, TT = TA + 1;
  const int64_t t0 = TT * part / p.n_parts, t1 = TT * (part + 1) / p.n_parts;
  const int nw = t1 - t0 > wave ? (int)((t1 - t0 - wave + 3) / 4) : 0;
  const int64_t nblk = (L + CAD_KV_BLOCK - 1) / CAD_KV_BLOCK;  // cached blocks of the sequence
  const int32_t* table = p.kv.table + (int64_t)p.rm.trow[b] * p.kv.max_blocks;
  const int64_t kv_blk_stride = (int64_t)p.hkv * CAD_KV_BLOCK * HD;
  const int64_t coff = (int64_t)p.rm.cidx[b] * p.kv.cache_stride + (int64_t)kvh * CAD_KV_BLOCK * HD;
  const bf16_t* kbase = (const bf16_t*)p.kv.k + coff;
  const bf16_t* vbase = (const bf16_t*)p.kv.v + coff;
  const int64_t srow0 = p.rm.pstart[b];  // span workspace row of key L (64-row padded region)

  f32x4 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -1e30f, l_run = 0.f;
  constexpr int QLDS = HD + 8;
  __shared__ __attribute__((aligned(16))) f16_t sq[2][16 * QLDS];

  {
    auto tile_of = [&](int i) -> int64_t { return t0 + wave + 4 * (int64_t)min(i, nw - 1); };
    // block ids of tile i: lanes with bit 0 clear read its first block, the
    // others its second (indices clamped to the sequence's cached blocks;
    // the span tile reads entry 0 and ignores it)
    auto ids_of = [&](int i) -> int32_t {
      const int64_t t = tile_of(i);
      const int64_t bi = t < TA ? min(2 * t + (lane & 1), nblk - 1) : 0;
      return table[bi];
    };
    struct Buf {
      u32x4 k[2][DS];
      u32x4 v[DB];
    };
    // raw loads of tile i (unconditional: the source is chosen by address).
    // Base pointers are wave-uniform; lane offsets (elements) are fixed per
    // lane: K [16 keys][HD] per cache block, V [HD][16] per cache block,
    // span K [row][hkv][HD], span V [hkv][HD][span_cap].
    const uint32_t ko_c = (uint32_t)(i16 * HD + 8 * g4);
    const uint32_t ko_s = (uint32_t)(i16 * p.hkv * HD + 8 * g4);
    const uint32_t vo_c = (uint32_t)(i16 * CAD_KV_BLOCK + 4 * g4);
    const uint32_t vo_s = (uint32_t)(i16 * p.kv.span_cap + 4 * g4);
    const f16_t* sk_base = p.kv.span_k + (srow0 * p.hkv + kvh) * HD;
    const f16_t* sv_base = p.kv.span_v + (int64_t)kvh * HD * p.kv.span_cap + srow0;
    auto issue = [&](Buf& bf, int i, int32_t ids) {
      const int64_t t = tile_of(i);
      const bool span = t >= TA;  // wave-uniform
      int64_t b0 = __builtin_amdgcn_readlane(ids, 0), b1 = __builtin_amdgcn_readlane(ids, 1);
      const bool ok = span || (b0 >= 0 && b0 < p.kv.num_blocks && b1 >= 0 && b1 < p.kv.num_blocks);
      if (!ok && p.status && lane == 0) atomicOr(p.status, (int32_t)CAD_DEV_BAD_BLOCK);
      if (!ok || span) b0 = b1 = 0;
      const uint32_t ko = span ? ko_s : ko_c;
      const uint32_t vo = span ? vo_s : vo_c;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint16_t* kp = span ? (const uint16_t*)(sk_base + (int64_t)16 * kb * p.hkv * HD)
                                  : (const uint16_t*)(kbase + (kb ? b1 : b0) * kv_blk_stride);
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) bf.k[kb][ds] = *(const u32x4*)(kp + ko + 32 * ds);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* vp0 = span ? (const uint16_t*)(sv_base + (int64_t)16 * db * p.kv.span_cap)
                                   : (const uint16_t*)(vbase + b0 * kv_blk_stride + 16 * db * CAD_KV_BLOCK);
        const uint16_t* vp1 = span ? vp0 + 16 : (const uint16_t*)(vbase + b1 * kv_blk_stride + 16 * db * CAD_KV_BLOCK);
        const u32x2 v0 = *(const u32x2*)(vp0 + vo);
        const u32x2 v1 = *(const u32x2*)(vp1 + vo);
        bf.v[db] = u32x4{v0[0], v0[1], v1[0], v1[1]};
      }
      return ok;
    };
    auto compute = [&](Buf& bf, int i, bool ok) {
      const int64_t t = tile_of(i);
      const bool span = t >= TA;
      // keys of the tile a query may see: [0, lim) relative to the tile start
      const int vlim = !ok ? 0 : span ? n_rows : (int)min<int64_t>(L - t * DEC_KT, DEC_KT);
      const int lim = span ? min(vlim, k_local + 1) : vlim;
      if (vlim < DEC_KT) {
        // zero V of keys past the range (stale slots may hold anything; P is 0 there)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int k0 = (w < 2 ? 0 : 16) + 4 * g4 + 2 * (w & 1);  // keys of the two halves of word w
            const uint32_t keep = (k0 + 1 < vlim) ? 0xFFFFFFFFu : (k0 < vlim ? 0x0000FFFFu : 0u);
            bf.v[db][w] &= keep;
          }
      }
      f32x4 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const u32x4 kf = span ? bf.k[kb][ds] : bf16x8_to_f16x8(bf.k[kb][ds]);
          const u32x4 qh = *(const u32x4*)(&sq[0][i16 * QLDS + 32 * ds + 8 * g4]);
          const u32x4 qlo = *(const u32x4*)(&sq[1][i16 * QLDS + 32 * ds + 8 * g4]);
          s[kb] = mfma16(kf, qh, s[kb]);
          s[kb] = mfma16(kf, qlo, s[kb]);
        }
      }
      if (lim < DEC_KT) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * kb + 4 * g4 + r >= lim) s[kb][r] = -INFINITY;
      }
      const float m4 = fmaxf(fmaxf(max_raw(s[0][0], s[0][1], p.pos_inf), max_raw(s[0][2], s[0][3], p.pos_inf)),
                             fmaxf(max_raw(s[1][0], s[1][1], p.pos_inf), max_raw(s[1][2], s[1][3], p.pos_inf)));
      const float mx = max_col4(m4, p.pos_inf) * p.scale_log2;
      if (__ballot(mx > m_run + FA_LAZY)) {  // wave-uniform rescale
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < DB; ++d) o[d] *= alpha;
      }
      const float nm = -m_run;
      const f16x2 ones = {(f16_t)1.0f, (f16_t)1.0f};
      float psum = 0.f;
      uint32_t pk[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], p.scale_log2, nm));
        const f16x2 e01 = {(f16_t)e[0], (f16_t)e[1]};
        const f16x2 e23 = {(f16_t)e[2], (f16_t)e[3]};
        psum = __builtin_amdgcn_fdot2(e01, ones, psum, false);
        psum = __builtin_amdgcn_fdot2(e23, ones, psum, false);
        pk[2 * kb] = __builtin_bit_cast(uint32_t, e01);
        pk[2 * kb + 1] = __builtin_bit_cast(uint32_t, e23);
      }
      l_run += psum;
      const u32x4 pf = {pk[0], pk[1], pk[2], pk[3]};
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x4 vf = span ? bf.v[db] : bf16x8_to_f16x8(bf.v[db]);
        o[db] = mfma16(vf, pf, o[db]);
      }
    };
    // tile i is computed while tile i + 1 is loaded; block ids run two
    // tiles ahead.  Loads past the wave's last tile re-read that tile
    // (clamped index: cache hits, never used).
    Buf A, B;
    int32_t idE = nw > 0 ? ids_of(0) : 0, idO = nw > 0 ? ids_of(1) : 0;
    // the work-group's q columns (hi and lo planes), shared by the four waves
    // through LDS: sq[plane][column][HD] (zero for columns past R); staged
    // while the first block ids are in flight, and the first tile is
    // requested before the barrier
    for (int c = tid; c < 2 * 16 * (HD / 8); c += 256) {
      const int pl = c / (16 * (HD / 8)), col = (c / (HD / 8)) % 16, c8 = c % (HD / 8);
      const bool okc = col < R;
      const int64_t row = (int64_t)(p.rm.start[b] + (okc ? col / p.G : 0)) * p.hq + kvh * p.G + (okc ? col % p.G : 0);
      const f16_t* src = (const f16_t*)(pl ? p.q_lo : p.q) + row * HD + 8 * c8;
      *(u32x4*)(&sq[pl][col * QLDS + 8 * c8]) = okc ? *(const u32x4*)src : u32x4{0u, 0u, 0u, 0u};
    }
    bool okA = nw > 0 ? issue(A, 0, idE) : false, okB = true;
    if (nw > 0) idE = ids_of(2);
    __syncthreads();
    for (int i = 0; i < nw; i += 2) {
      okB = issue(B, i + 1, idO);
      idO = ids_of(i + 3);
      compute(A, i, okA);
      if (i + 1 >= nw) break;
      okA = issue(A, i + 2, idE);
      idE = ids_of(i + 4);
      compute(B, i + 1, okB);
    }
  }
  // combine the four waves: (m, l) per query column and O^T
  __shared__ float sm[4][16], sl[4][16];
  __shared__ float so[4][16][HD + 4];
  float l = l_run;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (g4 == 0) {
    sm[wave][i16] = m_run;
    sl[wave][i16] = l;
  }
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) so[wave][i16][16 * db + 4 * g4 + r] = o[db][r];
  __syncthreads();
  // thread -> (query column q, dims d0 .. d0 + HD / 16 - 1)
  const int q = tid >> 4, d0 = (tid & 15) * (HD / 16);
  float m = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    if (sl[w][q] > 0.f) m = fmaxf(m, sm[w][q]);
  float wt[4], den = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wt[w] = sl[w][q] > 0.f ? __builtin_amdgcn_exp2f(sm[w][q] - m) : 0.f;
    den += wt[w] * sl[w][q];
  }
  if (q >= R) return;
  const int kq = q / p.G;
  const int64_t orow = (int64_t)(p.rm.start[b] + kq) * p.hq + kvh * p.G + q % p.G;
  if (p.n_parts == 1) {
    const float inv = den > 0.f ? 1.f / den : 0.f;
    bf16_t* out = (bf16_t*)p.out + orow * HD;
    bf16_t* out_lo = (bf16_t*)p.out_lo + orow * HD;
#pragma unroll
    for (int j = 0; j < HD / 16; ++j) {
      const int d = d0 + j;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) v += wt[w] * so[w][q][d];
      split_bf16(v * inv, out[d], out_lo[d]);
    }
  } else {
    const int64_t qi = (int64_t)part * p.rows * p.hq + orow;
    float* po = p.part_o + qi * HD;
#pragma unroll
    for (int j = 0; j < HD / 16; ++j) {
      const int d = d0 + j;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) v += wt[w] * so[w][q][d];
      po[d] = v;
    }
    if ((tid & 15) == 0) {
      p.part_ml[qi * 2 + 0] = den > 0.f ? m : -1e30f;
      p.part_ml[qi * 2 + 1] = den;
    }
  }
}

// log-sum-exp merge of the partitions (base-2 exponent, as produced above),
// written as bf16 hi / lo planes.  One work-group per (row, head): the
// partition weights 2^(m_p - m) (0 for a partition that saw no key) are
// formed once in LDS; with many partitions four thread groups each sum one
// quarter of them (eight loads in flight per thread) for the output
// dimension they own, and the quarters are added in order.
constexpr int MERGE_MAX_PARTS = 512;
constexpr int MERGE_GROUPS = 4;
__global__ void __launch_bounds__(128 * MERGE_GROUPS) k_attn_merge(const float* __restrict__ part_o,
                                                                   const float* __restrict__ part_ml, int n_parts,
                                                                   int64_t nq, int hd, bf16_t* __restrict__ out,
                                                                   bf16_t* __restrict__ out_lo) {
  __shared__ float sw[MERGE_MAX_PARTS], sl[MERGE_MAX_PARTS];
  __shared__ float red[MERGE_GROUPS * 2];
  __shared__ float snum[MERGE_GROUPS][128];
  const int64_t qi = blockIdx.x;
  const int t = threadIdx.x, nt = blockDim.x;
  const int ng = nt / 128, grp = t / 128, d = t % 128;
  const int q0 = n_parts * grp / ng, q1 = n_parts * (grp + 1) / ng;
  // the first MP partial outputs of this thread's range are loaded before
  // anything else (they do not depend on the weights)
  constexpr int MP = 16;
  const float* po = part_o + qi * hd + min(d, hd - 1);
  const int64_t stride = nq * hd;
  float ov0[MP];
#pragma unroll
  for (int u = 0; u < MP; ++u) ov0[u] = po[(int64_t)max(min(q0 + u, q1 - 1), 0) * stride];
  // maximum over partitions with a positive sum
  float mloc = -INFINITY;
  for (int pp = t; pp < n_parts; pp += nt) {
    const float2 ml = *(const float2*)(part_ml + ((int64_t)pp * nq + qi) * 2);
    sw[pp] = ml.y > 0.f ? ml.x : -INFINITY;
    sl[pp] = ml.y;
    mloc = fmaxf(mloc, sw[pp]);
  }
  for (int o = 32; o > 0; o >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o));
  if ((t & 63) == 0) red[t >> 6] = mloc;
  __syncthreads();
  float m = red[0];
  for (int w = 1; w < nt / 64; ++w) m = fmaxf(m, red[w]);
  for (int pp = t; pp < n_parts; pp += nt) sw[pp] = sw[pp] == -INFINITY ? 0.f : exp2f(sw[pp] - m);
  __syncthreads();
  // denominator: sum of w_p * l_p in partition order (every thread the same)
  float den = 0.f;
  for (int pp = 0; pp < n_parts; ++pp) den += sw[pp] * sl[pp];
  float num = 0.f;
  if (d < hd) {
#pragma unroll
    for (int u = 0; u < MP; ++u)
      if (q0 + u < q1) num += sw[q0 + u] * ov0[u];
    for (int pp = q0 + MP; pp < q1; pp += 8) {
      float ov[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) ov[u] = po[(int64_t)min(pp + u, q1 - 1) * stride];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (pp + u < q1) num += sw[pp + u] * ov[u];
    }
    snum[grp][d] = num;
  }
  __syncthreads();
  if (grp == 0 && d < hd) {
    float tot = snum[0][d];
    for (int g2 = 1; g2 < ng; ++g2) tot += snum[g2][d];
    split_bf16(den > 0.f ? tot / den : 0.f, out[qi * hd + d], out_lo[qi * hd + d]);
  }
}

// The same merge for at most NP <= MERGE_SMALL partitions (long spans): one
// thread per output element of four (row, head) pairs per work-group; each
// thread loads every partition's (max, sum) and its own partial values at
// once (no LDS, no barrier), forms the weights 2^(m_p - m) and adds the
// partitions in order.
constexpr int MERGE_SMALL = 16;
template <int NP>
__global__ void __launch_bounds__(512) k_attn_merge_small(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml, int n_parts,
                                                          int64_t nq, int hd, bf16_t* __restrict__ out,
                                                          bf16_t* __restrict__ out_lo) {
  const int64_t qi = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 7);
  const int d = threadIdx.x & 127;
  if (qi >= nq || d >= hd) return;
  float2 ml[NP];
  float ov[NP];
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const int q = min(pp, n_parts - 1);
    ml[pp] = *(const float2*)(part_ml + ((int64_t)q * nq + qi) * 2);
    ov[pp] = part_o[((int64_t)q * nq + qi) * hd + d];
  }
  float m = -INFINITY;
#pragma unroll
  for (int pp = 0; pp < NP; ++pp)
    if (pp < n_parts && ml[pp].y > 0.f) m = fmaxf(m, ml[pp].x);
  float den = 0.f, num = 0.f;
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    if (pp < n_parts && ml[pp].y > 0.f) {
      const float w = exp2f(ml[pp].x - m);
      den += w * ml[pp].y;
      num += w * ov[pp];
    }
  }
  split_bf16(den > 0.f ? num / den : 0.f, out[qi * hd + d], out_lo[qi * hd + d]);
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
  const float* kc = (const float*)p.kv.k + (int64_t)p.rm.cidx[b] * p.kv.cache_stride;
  const float* vc = (const float*)p.kv.v + (int64_t)p.rm.cidx[b] * p.kv.cache_stride;
  const int32_t* table = p.kv.table + (int64_t)p.rm.trow[b] * p.kv.max_blocks;
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

// the short-span kernel serves calls whose sequences all have at most 16
// query rows per KV head
inline bool attn_short(int max_seq_rows, int G) { return (int64_t)max_seq_rows * G <= 16; }
constexpr int DEC_TARGET_WGS = 256;  // short-span kernel: about one work-group per CU (measured: 512 ran 2 us slower at N = 1)

int attention_parts(int rows, int n_seq, int hq, int hkv, int64_t max_cache_keys, int max_seq_rows) {
  // partitions of each query tile's key axis: about one work-group per
  // compute unit (256 CUs; two for the four-wave shape)
  // together with the query tiles, at least 256 cached keys each, at least one
  const int G = hq / hkv;
  if (attn_short(max_seq_rows, G)) {
    const int base = n_seq * hkv;
    int parts = (DEC_TARGET_WGS + base - 1) / base;
    const int64_t cap = max_cache_keys / 256;
    if (parts > cap) parts = (int)cap;
    if (parts > MERGE_MAX_PARTS) parts = MERGE_MAX_PARTS;
    return parts < 1 ? 1 : parts;
  }
  const int qt = attn_qt(rows * G, n_seq);
  const int tiles = (rows * G + qt - 1) / qt;
  const int base = hkv * tiles;
  const int target = qt == 64 ? 512 : 256;
  int parts = (target + base - 1) / base;
  const int64_t cap = max_cache_keys / 256;
  if (parts > cap) parts = (int)cap;
  if (parts > MERGE_MAX_PARTS) parts = MERGE_MAX_PARTS;
  return parts < 1 ? 1 : parts;
}

hipError_t launch_attention(int dtype, const void* q, const void* q_lo, int rows, int hq, int hkv, int hd,
                            const RowMap& rm, KVView kv, int n_parts,
                            float* part_o, float* part_ml, void* out, void* out_lo, int32_t* status,
                            hipStream_t s) {
  AttnArgs a;
  a.q = q;
  a.q_lo = q_lo;
  a.rows = rows;
  a.hq = hq;
  a.hkv = hkv;
  a.G = hq / hkv;
  a.rm = rm;
  a.kv = kv;
  a.n_parts = n_parts;
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.out = out;
  a.out_lo = out_lo;
  a.status = status;
  a.scale_log2 = 1.4426950408889634f / sqrtf((float)hd);
  a.pos_inf = INFINITY;
  if (dtype == CAD_F32) {
    hipLaunchKernelGGL(k_attn_f32, dim3(rows, hq), dim3(64), 0, s, a, hd);
    return hipGetLastError();
  }
  int max_seq_rows = 0;
  for (int b = 0; b < rm.n_seq; ++b) max_seq_rows = max(max_seq_rows, rm.start[b + 1] - rm.start[b]);
  if (attn_short(max_seq_rows, a.G)) {
    const int64_t wgs = (int64_t)rm.n_seq * hkv * n_parts;
    if (wgs > INT32_MAX || (hd != 64 && hd != 128)) return hipErrorInvalidValue;
    if (hd == 64)
      hipLaunchKernelGGL((k_attn_dec<64>), dim3((unsigned)wgs), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_attn_dec<128>), dim3((unsigned)wgs), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const int qt = attn_qt(rows * a.G, rm.n_seq);
  int nt = 0;
  a.tstart[0] = 0;
  for (int b = 0; b < rm.n_seq; ++b) {
    const int R = (rm.start[b + 1] - rm.start[b]) * a.G;
    nt += (R + qt - 1) / qt;
    a.tstart[b + 1] = nt;
  }
  dim3 grid(nt, hkv, n_parts);
  if (hd == 64 && qt == 64)
    hipLaunchKernelGGL((k_attn_bf16<64, 4, 1>), grid, dim3(256), 0, s, a);
  else if (hd == 64)
    hipLaunchKernelGGL((k_attn_bf16<64, 8, 2>), grid, dim3(512), 0, s, a);
  else if (qt == 64)
    hipLaunchKernelGGL((k_attn_bf16<128, 4, 1>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_attn_bf16<128, 8, 2>), grid, dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attention_merge(const float* part_o, const float* part_ml, int n_parts, int rows,
                                  int hq, int hd, void* out, void* out_lo, hipStream_t s) {
  const int64_t nq = (int64_t)rows * hq;
  if (n_parts > MERGE_MAX_PARTS || hd > 128) return hipErrorInvalidValue;
  if (n_parts <= MERGE_SMALL) {
    const dim3 grid((unsigned)((nq + 3) / 4));
    if (n_parts <= 4)
      hipLaunchKernelGGL(k_attn_merge_small<4>, grid, dim3(512), 0, s, part_o, part_ml, n_parts, nq, hd,
                         (bf16_t*)out, (bf16_t*)out_lo);
    else if (n_parts <= 8)
      hipLaunchKernelGGL(k_attn_merge_small<8>, grid, dim3(512), 0, s, part_o, part_ml, n_parts, nq, hd,
                         (bf16_t*)out, (bf16_t*)out_lo);
    else
      hipLaunchKernelGGL(k_attn_merge_small<16>, grid, dim3(512), 0, s, part_o, part_ml, n_parts, nq, hd,
                         (bf16_t*)out, (bf16_t*)out_lo);
    return hipGetLastError();
  }
  const int groups = n_parts >= 16 ? MERGE_GROUPS : 1;
  hipLaunchKernelGGL(k_attn_merge, dim3((unsigned)nq), dim3(128 * groups), 0, s, part_o, part_ml, n_parts, nq, hd,
                     (bf16_t*)out, (bf16_t*)out_lo);
  return hipGetLastError();
}

}  // namespace cad
