// rz_calib.hip -- measurement support, not part of the method: the rate at
// which this chip's matrix cores run the learner GEMMs' instruction
// (v_mfma_f32_32x32x16_bf16) under its own clock and power management, with
// no global memory traffic at all.
//
// Each workgroup is four waves, one per SIMD.  A wave keeps sixteen 32 x 32
// fp32 accumulators (a 128 x 128 block: the four-wave layout of the 256 x 256
// tile, whose MFMA stream per SIMD equals that of the two waves of the
// library's eight-wave tile) and eight fragments of each operand;
// K step s feeds accumulator (mi, ni) with A fragment (s + mi) % 8 and B
// fragment (s + 3 ni) % 8, so successive MFMAs see new operand values as in
// a GEMM.
// from_lds = 0 keeps the fragments in registers; from_lds = 1 reads the
// step's four A and four B fragments from LDS before its sixteen MFMAs
// (the GEMM's LDS read volume per MFMA, without its global loads).
// data = 1 fills the fragments with bf16 values from an integer hash
// (magnitudes up to about 2, both signs); data = 0 with zeros, which
// switch no multiplier bits: the difference shows what the operands' values
// cost in power.
#include "../../include/rz.h"
#include "rz_gemm.h"

namespace rz {
namespace {

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  // an integer finaliser (xorshift-multiply), to spread the bits
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// eight bf16 values: sign and mantissa from the hash, exponent 126 or 127
// (magnitudes in [0.5, 2))
__device__ __forceinline__ u32x4 hashed_frag(uint32_t salt) {
  u32x4 v;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t h = mix32(salt * 4u + (uint32_t)w);
    const uint32_t lo = (h & 0x807Fu) | ((126u + ((h >> 7) & 1u)) << 7);
    const uint32_t hi = ((h >> 16) & 0x807Fu) | ((126u + ((h >> 23) & 1u)) << 7);
    v[w] = lo | (hi << 16);
  }
  return v;
}

template <int kLds>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_mfma_ceiling(int data, int64_t iters, float* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) char lds[kLds ? 4 * 16384 : 16];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  u32x4 fa[8], fb[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const uint32_t base = ((uint32_t)blockIdx.x * 256u + threadIdx.x) * 16u;
    fa[f] = data ? hashed_frag(base + f) : u32x4{0u, 0u, 0u, 0u};
    fb[f] = data ? hashed_frag(base + 8 + f) : u32x4{0u, 0u, 0u, 0u};
  }
  // LDS: each wave owns 16 KB, fragment f of operand o of lane l at
  // ((o * 8 + f) * 64 + l) * 16 (consecutive lanes, consecutive 16 bytes)
  char* mine = lds + (kLds ? wid * 16384 : 0);
  if constexpr (kLds) {
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      *reinterpret_cast<u32x4*>(mine + ((0 * 8 + f) * 64 + lane) * 16) = fa[f];
      *reinterpret_cast<u32x4*>(mine + ((1 * 8 + f) * 64 + lane) * 16) = fb[f];
    }
    __syncthreads();
  }
  f32x16 acc[kTM][kTN];
#pragma unroll
  for (int mi = 0; mi < kTM; ++mi)
#pragma unroll
    for (int ni = 0; ni < kTN; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
  const int wbase = kLds ? wid * 16384 : 0;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      // an opaque offset into the LDS array every step: each step issues
      // its eight reads (ds_read_b128), none merged with another step's
      int off = wbase;
      asm volatile("" : "+v"(off));
      const char* src = lds + off;
      u32x4 a[kTM], b[kTN];
#pragma unroll
      for (int mi = 0; mi < kTM; ++mi)
        a[mi] = kLds ? *reinterpret_cast<const u32x4*>(src + ((0 * 8 + (s + mi) % 8) * 64 + lane) * 16)
                     : fa[(s + mi) % 8];
#pragma unroll
      for (int ni = 0; ni < kTN; ++ni)
        b[ni] = kLds ? *reinterpret_cast<const u32x4*>(src + ((1 * 8 + (s + 3 * ni) % 8) * 64 + lane) * 16)
                     : fb[(s + 3 * ni) % 8];
#pragma unroll
      for (int mi = 0; mi < kTM; ++mi)
#pragma unroll
        for (int ni = 0; ni < kTN; ++ni) mfma_step(acc[mi][ni], a[mi], b[ni], (const bf16*)nullptr);
    }
  }
  float t = 0.f;
#pragma unroll
  for (int mi = 0; mi < kTM; ++mi)
#pragma unroll
    for (int ni = 0; ni < kTN; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) t += acc[mi][ni][r];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = t;
}

}  // namespace
}  // namespace rz

extern "C" rz_status rz_calibrate_mfma(int32_t data, int32_t from_lds,
                                       int32_t n_workgroups, int64_t iters,
                                       float* sink, hipStream_t stream) {
  if ((data != 0 && data != 1) || (from_lds != 0 && from_lds != 1) ||
      n_workgroups < 1 || n_workgroups > (1 << 20) || iters < 0 || !sink)
    return RZ_ERR_INVALID_ARG;
  if (from_lds)
    rz::k_mfma_ceiling<1><<<n_workgroups, 256, 0, stream>>>(data, iters, sink);
  else
    rz::k_mfma_ceiling<0><<<n_workgroups, 256, 0, stream>>>(data, iters, sink);
  return hipGetLastError() == hipSuccess ? RZ_OK : RZ_ERR_HIP;
}
