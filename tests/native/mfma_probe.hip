// mfma_probe.hip -- test-only probe of one bare FP8 matrix-core instruction (gfx950).
//
// The FP8 indexer score kernel forms its q.k dot products with
// v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 operands, unit scales), and the tolerance its
// tests apply models how that instruction adds the 128 products of a dot product. This
// probe runs the instruction alone -- one wave, one 16 x 16 x 128 tile, zero accumulator,
// no staging, no epilogue -- so the model can be measured on the instruction itself
// instead of on the kernel it bounds:
//
//     c[m * 16 + n] = sum_d a[m * 128 + d] * b[n * 128 + d]      (m, n < 16, d < 128)
//
// Lane l holds the 32 bytes d = 32 (l / 16) .. 32 (l / 16) + 31 of A row l % 16 and of
// B column l % 16, the same slice in the same lane positions for both operands, and
// receives rows 4 (l / 16) .. 4 (l / 16) + 3 of output column l % 16.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64) void mfma_probe_kernel(const uint8_t* __restrict__ a,
                                                        const uint8_t* __restrict__ b,
                                                        float* __restrict__ c) {
  const int l = threadIdx.x;
  const int r = l % 16, g = l / 16;
  const int4* pa = reinterpret_cast<const int4*>(a + r * 128 + g * 32);
  const int4* pb = reinterpret_cast<const int4*>(b + r * 128 + g * 32);
  int4 a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
  v8i va = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
  v8i vb = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
  v4f zero = {0.f, 0.f, 0.f, 0.f};
  v4f acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, vb, zero, 0, 0, 0, 0, 0, 0);
  for (int i = 0; i < 4; ++i) c[(4 * g + i) * 16 + r] = acc[i];
}

}  // namespace

// a: 16 x 128 E4M3 codes (row-major, device, 16-byte aligned); b: 16 x 128 E4M3 codes
// (key-major: row n is column n of the B operand, device, 16-byte aligned); c: 16 x 16
// floats (device). One wave on the given stream; returns the launch's hipError_t.
extern "C" int mfma_probe_tile(const uint8_t* a, const uint8_t* b, float* c, hipStream_t stream) {
  if (!a || !b || !c) return hipErrorInvalidValue;
  if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(1), dim3(64), 0, stream, a, b, c);
  return static_cast<int>(hipGetLastError());
}
