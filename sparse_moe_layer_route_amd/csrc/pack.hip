// Fragment-major ("MFMA16") packing of bf16 weight matrices.
//
// A matrix W [R][K] (k contiguous) is stored as [ceil(R/16)][ceil(K/32)][64][8]:
// fragment (t, s) is the 1 KiB operand of one v_mfma_f32_16x16x32_bf16 for
// rows 16t..16t+15 and k 32s..32s+31, lane l holding row 16t + l%16 and the
// eight k values from 32s + 8*(l/16), zero past R or K.  A wave then loads a
// whole fragment with one contiguous 1 KiB access (16 bytes per lane), and the
// fragments of a row strip follow each other along k, so a wave walking k
// streams one contiguous range; the row-major form reads 64 bytes from each of
// 16 rows at the row stride instead, which HBM serves at a lower rate.
#include <algorithm>

#include "common.h"

namespace moe {

// One thread per 16-byte lane slot of the destination (K % 8 == 0, so a slot
// is either wholly inside K or wholly past it).
__global__ void __launch_bounds__(256)
pack_mfma16_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int R, int K,
                   int RT, int KS, int64_t slots) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < slots;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(i & 63);
    const int64_t f = i >> 6;                 // fragment index over (g, t, s)
    const int s = (int)(f % KS);
    const int64_t gt = f / KS;
    const int t = (int)(gt % RT);
    const int64_t g = gt / RT;
    const int row = 16 * t + (l & 15), k0 = 32 * s + 8 * (l >> 4);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < R && k0 < K)
      v = *reinterpret_cast<const uint4*>(src + (g * R + row) * (int64_t)K + k0);
    *reinterpret_cast<uint4*>(dst + i * 8) = v;
  }
}

int64_t packed_elems(int R, int K) {
  return (int64_t)((R + 15) / 16) * 16 * (int64_t)((K + 31) / 32) * 32;
}

hipError_t launch_pack_mfma16(int G, int R, int K, const void* src, void* dst, hipStream_t s) {
  const int RT = (R + 15) / 16, KS = (K + 31) / 32;
  const int64_t slots = (int64_t)G * RT * KS * 64;
  const int64_t want = (slots + 255) / 256;
  const int blocks = (int)std::min<int64_t>(want, 1 << 16);
  pack_mfma16_kernel<<<blocks, 256, 0, s>>>((const uint16_t*)src, (uint16_t*)dst, R, K, RT, KS,
                                            slots);
  return hipGetLastError();
}

}  // namespace moe
