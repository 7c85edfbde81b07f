// indexer_scores.hip -- FP8 indexer score producer for the exact Top-K selector (gfx950).
//
// Computes, for query row t and key s, the DSA-style indexer score of page "LiteTopK:
// Exploiting the Curse of Dimensionality for a Fused Indexer-TopK Kernel ..." (section
// 核心公式, Eq. (1)):
//
//     I[t, s] = sum_h w[t, h] * ReLU(q[t, h, :] . k[s, :])        for s <  L_t
//     I[t, s] = -inf                                               for s >= L_t
//
// with q and k in FP8 (OCP E4M3) and w in FP32. This is the score matrix the selector
// consumes: ragged rows with a -inf suffix. The pages chain the selector behind an FP8
// multi-query score kernel in one graph (page "几何平均快 1.55 倍，但短行采样会输：腾讯怎么测精确
// Top-K", section "框架轨迹"); this kernel plays that part.
//
// Design (CDNA4, wave64). The q.k products are a dense contraction over the head
// dimension D = 128, so they run on the matrix cores: one v_mfma_f32_16x16x128_f8f6f4 gives
// the dot products of 16 heads of one query with 16 keys. Each wave keeps the A operands
// (its queries' heads, 32 B per lane per 16-head group) in registers for the whole key
// range; the workgroup streams its 4096-key range through LDS in 64-key blocks, and the
// waves take their 16-key B operands from there. The ReLU, the weighting by w and the sum
// over heads are VALU work on the accumulators (two VALU ops per head and key, about as
// many cycles as the MFMA that produced them; the library is built with the MFMA results
// in ordinary VGPRs so that no accumulator-register copies are added):
//   * lane (g = lane / 16, c = lane % 16) of an MFMA output holds heads 4g..4g+3 of the
//     16-head group for key c; it folds its 4 heads of every group into one partial sum;
//   * four 16-key steps (64 keys) are then combined across the four lane groups by a
//     two-step butterfly (lane ^ 32, lane ^ 16) that leaves lane l with the total for
//     key 64-block base + l, so every wave writes 256 contiguous bytes per query.
// The A and B operands hold the same 32-byte slice of D in the same lane positions, so the
// contraction is correct whatever order the instruction walks D in internally.
// Products of two E4M3 values are exact. The matrix core adds them in groups of 8 adjacent
// products, each first truncated toward zero to a multiple of 2^(X - 13), where X is the
// largest exponent sum e_q + e_k over the group's nonzero products (measured on the bare
// gfx950 instruction); group sums, accumulator and head sum round in FP32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "topk_exact.h"

int topk_record_error(int code, const char* text);  // defined with the selector (error text)

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int WAVES = 4;                  // waves per workgroup
constexpr int QPW = 2;                    // queries per wave
constexpr int QPB = WAVES * QPW;          // queries per workgroup
constexpr int DIM = 128;                  // head dimension (one MFMA K step)
constexpr int KEYS_PER_BLOCK = 64;        // keys per wave iteration (4 MFMA column tiles)
constexpr int KEYS_PER_WG = 4096;         // key range of one workgroup

__device__ __forceinline__ v8i load32(const uint8_t* p) {
  const int4* v = reinterpret_cast<const int4*>(p);
  int4 a = v[0], b = v[1];
  v8i r = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  return r;
}

// ReLU on the bit pattern: a float with its sign bit set is a negative int32 and becomes
// +0 under a signed max, every other value is kept. One VALU op, where fmaxf(x, 0) costs
// two (the IEEE-mode max first canonicalizes its input).
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// The lane's partial sum over its 4 heads of each 16-head group for one 16-key step of one
// query, from that step's HG MFMA accumulators.
template <int HG>
__device__ __forceinline__ float weighted_relu_sum(const v4f (&acc)[HG], const float (&wl)[HG][4]) {
  float p = 0.f;
#pragma unroll
  for (int hg = 0; hg < HG; ++hg)
#pragma unroll
    for (int r = 0; r < 4; ++r) p = fmaf(wl[hg][r], relu(acc[hg][r]), p);
  return p;
}

// Lane l of the wave holds p[j] = its partial for key base + 16 j + (l % 16) from lane group
// g = l / 16. Returns the sum over the four lane groups for key base + l.
__device__ __forceinline__ float reduce_scatter4(const float (&p)[4], int lane) {
  const bool hi2 = (lane >> 5) & 1;  // g >> 1
  const bool hi1 = (lane >> 4) & 1;  // g & 1
  float send_a = hi2 ? p[0] : p[2], send_b = hi2 ? p[1] : p[3];
  float keep_a = hi2 ? p[2] : p[0], keep_b = hi2 ? p[3] : p[1];
  float q0 = keep_a + __shfl_xor(send_a, 32);
  float q1 = keep_b + __shfl_xor(send_b, 32);
  float send = hi1 ? q0 : q1, keep = hi1 ? q1 : q0;
  return keep + __shfl_xor(send, 16);
}

// Shared-memory staging of the key stream: every wave of a workgroup needs the same 16-key
// B operands, so the workgroup copies each 64-key block (8 KB) into LDS once, one block
// ahead of its use (double buffer), and the waves read their operands from there. Rows
// are padded from 128 to 144 bytes so that the 16 lanes reading one 16-byte slice of 16
// different keys hit 16 disjoint groups of 4 banks.
constexpr int PITCH = 144;

template <int HG>
__global__ __launch_bounds__(WAVES * 64) void indexer_scores_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const float* __restrict__ w,
    const int32_t* __restrict__ row_len, int T, int S, int n_qgroups, float* __restrict__ out) {
  constexpr int H = HG * 16;
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][KEYS_PER_BLOCK * PITCH];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int qg = blockIdx.x % n_qgroups;
  const int kc = blockIdx.x / n_qgroups;
  const int s_begin = kc * KEYS_PER_WG;
  const int s_end = min(S, s_begin + KEYS_PER_WG);

  // Queries of this wave, their lengths and operands.
  int t[QPW], L[QPW];
  v8i a[QPW][HG];
  float wl[QPW][HG][4];
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    t[i] = qg * QPB + wave * QPW + i;
    const bool live = t[i] < T;
    const int tt = live ? t[i] : 0;
    // The length is the same for every lane; readfirstlane makes the branches on it uniform.
    L[i] = __builtin_amdgcn_readfirstlane(live ? min(max(row_len[tt], 0), S) : 0);
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      a[i][hg] = load32(q + ((size_t)tt * H + hg * 16 + c) * DIM + g * 32);
      const float4 wv = *reinterpret_cast<const float4*>(w + (size_t)tt * H + hg * 16 + 4 * g);
      wl[i][hg][0] = wv.x; wl[i][hg][1] = wv.y; wl[i][hg][2] = wv.z; wl[i][hg][3] = wv.w;
    }
  }
  int Lmax = 0;  // the wave's longest row: blocks past it only write -inf
#pragma unroll
  for (int i = 0; i < QPW; ++i) Lmax = max(Lmax, L[i]);
  const float ninf = -__builtin_inff();

  // Staging: thread tid copies bytes [part * 32, part * 32 + 32) of key (tid / 4) of a block.
  // Keys past S are read from row S - 1 (in bounds) and their scores are never stored.
  const int skey = tid >> 2, part = tid & 3;
  const int soff = skey * PITCH + part * 32;
  {
    const int4* src = reinterpret_cast<const int4*>(k + (size_t)min(s_begin + skey, S - 1) * DIM + part * 32);
    const int4 r0 = src[0], r1 = src[1];
    *reinterpret_cast<int4*>(&kbuf[0][soff]) = r0;
    *reinterpret_cast<int4*>(&kbuf[0][soff + 16]) = r1;
  }
  __syncthreads();

  int buf = 0;
  for (int s0 = s_begin; s0 < s_end; s0 += KEYS_PER_BLOCK) {
    // Fetch the next block into registers now; it goes to the other buffer after this
    // block's work, so its latency overlaps the matrix and vector work below.
    const int nxt = s0 + KEYS_PER_BLOCK;
    const bool more = nxt < s_end;
    int4 r0 = {0, 0, 0, 0}, r1 = {0, 0, 0, 0};
    if (more) {
      const int4* src = reinterpret_cast<const int4*>(k + (size_t)min(nxt + skey, S - 1) * DIM + part * 32);
      r0 = src[0];
      r1 = src[1];
    }
    float p[QPW][4];
#pragma unroll
    for (int i = 0; i < QPW; ++i) p[i][0] = p[i][1] = p[i][2] = p[i][3] = 0.f;
    if (s0 < Lmax) {
      // All 4 x QPW x HG products of the block first, then the epilogue: the matrix work of
      // later products overlaps the ReLU / weighting of earlier ones.
      v4f acc[4][QPW][HG];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint8_t* bp = &kbuf[buf][(16 * j + c) * PITCH + g * 32];
        const int4 x0 = *reinterpret_cast<const int4*>(bp), x1 = *reinterpret_cast<const int4*>(bp + 16);
        const v8i b = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int i = 0; i < QPW; ++i)
#pragma unroll
          for (int hg = 0; hg < HG; ++hg) {
            const v4f zero = {0.f, 0.f, 0.f, 0.f};
            acc[j][i][hg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i][hg], b, zero, 0, 0, 0, 0, 0, 0);
          }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < QPW; ++i) p[i][j] = weighted_relu_sum<HG>(acc[j][i], wl[i]);
#pragma unroll
      for (int i = 0; i < QPW; ++i)  // a query whose row ends before this block
        if (s0 >= L[i]) p[i][0] = p[i][1] = p[i][2] = p[i][3] = 0.f;
    }
    const int s = s0 + lane;
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      const float res = reduce_scatter4(p[i], lane);
      if (s < s_end && t[i] < T) out[(size_t)t[i] * S + s] = (s < L[i]) ? res : ninf;
    }
    if (more) {
      *reinterpret_cast<int4*>(&kbuf[buf ^ 1][soff]) = r0;
      *reinterpret_cast<int4*>(&kbuf[buf ^ 1][soff + 16]) = r1;
    }
    __syncthreads();
    buf ^= 1;
  }
}

}  // namespace

// Host-side checks of a score call (no launch); shared with the score + select chain.
__attribute__((visibility("hidden"))) int topk_indexer_check(const uint8_t* q, const uint8_t* k,
                                                            const float* w, const int32_t* row_len,
                                                            int64_t T, int64_t S, int32_t H, int32_t D,
                                                            const float* out) {
  if (T < 0) return topk_record_error(TOPK_ERR_BAD_SHAPE, "indexer: T is negative");
  // Key offsets are int arithmetic in the kernel: the last key chunk ends below INT32_MAX.
  if (S < 1 || S > (int64_t)INT32_MAX - KEYS_PER_WG)
    return topk_record_error(TOPK_ERR_BAD_SHAPE, "indexer: S outside [1, INT32_MAX - 4096]");
  if (T > INT32_MAX || (T > 0 && S > INT64_MAX / 4 / T))
    return topk_record_error(TOPK_ERR_BAD_SHAPE, "indexer: T outside [0, INT32_MAX] or T * S overflows");
  if (D != DIM) return topk_record_error(TOPK_ERR_BAD_ARG, "indexer: D must be 128");
  if (H != 16 && H != 32 && H != 48 && H != 64)
    return topk_record_error(TOPK_ERR_BAD_ARG, "indexer: H must be 16, 32, 48 or 64");
  if (T == 0) return TOPK_OK;
  if (!q || !k || !w || !row_len || !out)
    return topk_record_error(TOPK_ERR_NULL_POINTER, "indexer: null pointer argument");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)w) & 15)
    return topk_record_error(TOPK_ERR_BAD_ARG, "indexer: q, k and w must be 16-byte aligned");
  const int64_t n_qgroups = (T + QPB - 1) / QPB;
  const int64_t n_kchunks = (S + KEYS_PER_WG - 1) / KEYS_PER_WG;
  if (n_kchunks * n_qgroups > INT32_MAX) return topk_record_error(TOPK_ERR_BAD_SHAPE, "indexer: grid too large");
  return TOPK_OK;
}

// Enqueues the score kernel of a checked call (T > 0).
__attribute__((visibility("hidden"))) int topk_indexer_launch(const uint8_t* q, const uint8_t* k,
                                                             const float* w, const int32_t* row_len,
                                                             int64_t T, int64_t S, int32_t H, float* out,
                                                             hipStream_t stream) {
  const int n_qgroups = (int)((T + QPB - 1) / QPB);
  const int64_t n_kchunks = (S + KEYS_PER_WG - 1) / KEYS_PER_WG;
  dim3 grid((unsigned)(n_kchunks * n_qgroups)), block(WAVES * 64);
  switch (H) {
    case 16: indexer_scores_kernel<1><<<grid, block, 0, stream>>>(q, k, w, row_len, (int)T, (int)S, n_qgroups, out); break;
    case 32: indexer_scores_kernel<2><<<grid, block, 0, stream>>>(q, k, w, row_len, (int)T, (int)S, n_qgroups, out); break;
    case 48: indexer_scores_kernel<3><<<grid, block, 0, stream>>>(q, k, w, row_len, (int)T, (int)S, n_qgroups, out); break;
    default: indexer_scores_kernel<4><<<grid, block, 0, stream>>>(q, k, w, row_len, (int)T, (int)S, n_qgroups, out); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return topk_record_error(TOPK_ERR_HIP, hipGetErrorString(e));
  return TOPK_OK;
}

extern "C" int topk_indexer_scores(const uint8_t* q, const uint8_t* k, const float* w,
                                   const int32_t* row_len, int64_t T, int64_t S, int32_t H,
                                   int32_t D, float* out, hipStream_t stream) {
  topk_record_error(TOPK_OK, "");  // clears the error text
  const int rc = topk_indexer_check(q, k, w, row_len, T, S, H, D, out);
  if (rc != TOPK_OK || T == 0) return rc;
  return topk_indexer_launch(q, k, w, row_len, T, S, H, out, stream);
}
