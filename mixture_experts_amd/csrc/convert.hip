// Weight conversion MXFP4 -> the fp8 recipe's format: the DeepSeek-V4-Pro
// overview (lzwjava.github.io), convert.py entry: FP4 (e2m1fn) to FP8 (e4m3fn)
// without loss, with care for the scales.
//
// One workgroup per 128 x 128 block.  The block's scale is 2^(E - 127) with E the
// largest E8M0 byte of its 512 per-32 groups; an element with group byte b and e2m1
// value q becomes the e4m3 code of q * 2^(b - E) (nearest, ties to even).  Every
// e2m1 value is an e4m3 value, so the block is exact whenever its groups lie within
// 8 binades of E (0.5 * 2^-8 is e4m3's smallest subnormal); a block that is not is
// counted.
#include "kernels.h"

namespace moe {

namespace {

__global__ void zero_counter(int32_t* c) {
  if (threadIdx.x == 0) *c = 0;
}

// Thread t: row t / 2 of the block, columns 64 (t & 1) .. +64 (two groups of 32).
__global__ __launch_bounds__(256) void mxfp4_to_fp8_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ e8,
                                                           uint8_t* __restrict__ out, float* __restrict__ out_scale,
                                                           int32_t* __restrict__ inexact, int row_len) {
  __shared__ uint32_t wmax[4];
  const int bc = blockIdx.x, br = blockIdx.y, t = threadIdx.x;
  const int r = t >> 1, h = t & 1;
  const size_t row = size_t(br) * 128 + r;
  const int ngr = row_len / 32;
  const uint32_t s2 = *reinterpret_cast<const uint16_t*>(e8 + row * ngr + bc * 4 + 2 * h);   // groups 2h, 2h+1
  const uint32_t b0 = s2 & 0xffu, b1 = s2 >> 8;
  uint32_t m = max(b0, b1);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, uint32_t(__shfl_xor(int(m), off, 64)));
  if ((t & 63) == 0) wmax[t >> 6] = m;
  __syncthreads();
  const int E = int(max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])));
  bool exact = true;
  const uint8_t* src = q + row * (row_len / 2) + bc * 64 + 32 * h;
  uint8_t* dst = out + row * row_len + bc * 128 + 64 * h;
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const float sc = exp2i(max(int(gi ? b1 : b0) - E, -149));   // 2^(b - E), exact (or 2^-149 when lower)
    const uint4 w = *reinterpret_cast<const uint4*>(src + 16 * gi);
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {                  // 4 codes per output dword
      uint32_t packed = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t nib = (wd[i >> 1] >> (4 * (4 * (i & 1) + j))) & 15u;
        const float v = e2m1_to_f32(nib) * sc;     // exact: at most two significant bits
        const uint32_t c = f32_to_e4m3(v);
        exact &= e4m3_to_f32(c) == v;
        packed |= c << (8 * j);
      }
      o[i] = packed;
    }
    *reinterpret_cast<uint4*>(dst + 32 * gi) = uint4{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<uint4*>(dst + 32 * gi + 16) = uint4{o[4], o[5], o[6], o[7]};
  }
  const int all_exact = __syncthreads_and(int(exact));
  if (t == 0) {
    out_scale[size_t(br) * (row_len / 128) + bc] = exp2i(E - 127);
    if (inexact && !all_exact) atomicAdd(inexact, 1);
  }
}

}  // namespace

hipError_t launch_mxfp4_to_fp8(int64_t rows, int row_len, const void* q, const void* e8, void* out, float* out_scale,
                               int32_t* inexact, hipStream_t st) {
  if (inexact) zero_counter<<<1, 64, 0, st>>>(inexact);
  mxfp4_to_fp8_kernel<<<dim3(row_len / 128, unsigned(rows / 128)), 256, 0, st>>>(
      static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(e8), static_cast<uint8_t*>(out), out_scale, inexact,
      row_len);
  return hipGetLastError();
}

}  // namespace moe
