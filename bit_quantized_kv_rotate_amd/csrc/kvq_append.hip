// Write path of the rotated 4-bit KV cache: Walsh-Hadamard rotation, shared
// power-of-two (UE8M0) scale per 32 channels, E2M1 codes (or the E4M3
// comparator), stored into the paged layout; and the dequantiser used by
// tests.  Method: ROCm blog "UltraQuant on AMD Instinct", section "What is
// UltraQuant?" (rotation before the FP4 grid, one power-of-two scale per 32
// channels, 17 bytes per group).
//
// Built with -ffp-contract=off: every fp32 add, subtract and multiply of the
// rotation rounds once, in the documented order, so the stored codes are
// reproducible bit for bit.
#include "kvq_append_dev.h"

namespace kvq {
namespace {

// 1-D grid, the (KV head, tensor) pair fastest: the blocks that run together
// cover every head of the same tokens, so each token's bf16 row (all heads,
// contiguous) is read whole at once rather than one head at a time.  When the
// pair count n_ht is a multiple of 4, the four waves of a block take four
// consecutive pairs of the same tokens (1 KB of each token's row per block,
// and neighbouring heads' scale bytes, which share cache lines, written from
// one compute unit): the whole b32_l32k cache build 4.77 -> 5.19 TB/s against
// four consecutive token ranges of one pair per block.
template <int G>
__global__ __launch_bounds__(256) void append_kernel(const AppendParams p, unsigned n_ht) {
  unsigned ht, w;  // (KV head, tensor) pair, wave index within the pair's tokens
  if ((n_ht & 3u) == 0) {
    const unsigned q = n_ht >> 2;
    ht = (blockIdx.x % q) * 4 + (threadIdx.x >> 6);
    w = blockIdx.x / q;
  } else {
    ht = blockIdx.x % n_ht;
    w = (blockIdx.x / n_ht) * 4 + (threadIdx.x >> 6);
  }
  append_wave<G>(p, (int)w, (int)(ht % (unsigned)p.c.hkv), (int)(ht / (unsigned)p.c.hkv), threadIdx.x & 63);
}

struct DequantParams {
  CacheGeom c;
  const int32_t* slots;
  float* k_out;
  float* v_out;
};

__device__ __forceinline__ float e2m1_value(uint32_t code) {
  const uint32_t k = code & 7u;
  // 0, 0.5, 1, 1.5, 2, 3, 4, 6
  float v = (k < 4) ? 0.5f * (float)k : (float)(2u << ((k - 4) >> 1)) * ((k & 1) ? 1.5f : 1.0f);
  return (code & 8u) ? -v : v;
}

__device__ __forceinline__ float e4m3_value(uint32_t code) {
  const uint32_t e = (code >> 3) & 15u;
  const uint32_t m = code & 7u;
  float v;
  if (e == 15u && m == 7u)
    v = __builtin_nanf("");
  else if (e == 0u)
    v = ldexpf((float)m, -9);
  else
    v = ldexpf(1.0f + (float)m * 0.125f, (int)e - 7);
  return (code & 0x80u) ? -v : v;
}

__global__ __launch_bounds__(64) void dequant_kernel(const DequantParams p) {
  const int tid = threadIdx.x;
  const int n = blockIdx.x;
  const int h = blockIdx.y;
  const int tensor = blockIdx.z;
  const CacheGeom& c = p.c;
  const int slot = p.slots[n];
  const int page = slot / c.p;
  const int off = slot - page * c.p;
  const uint8_t* codes = (tensor == 0 ? c.kc : c.vc) + (int64_t)page * c.c_page + (int64_t)h * c.c_head;
  const uint8_t* scales = (tensor == 0 ? c.ks : c.vs) + (int64_t)page * c.s_page + (int64_t)h * c.s_head;
  float* out = (tensor == 0 ? p.k_out : p.v_out) + ((size_t)n * c.hkv + h) * c.d;
  for (int ch = tid; ch < c.d; ch += 64) {
    const int g = ch >> 5;
    const int byte = scales[(int64_t)g * c.p + off];
    float v;
    if (c.fmt == KVQ_FMT_FP4_E2M1) {
      const uint32_t pair = codes[((int64_t)g * c.p + off) * 16 + ((ch & 31) >> 1)];
      v = e2m1_value((ch & 1) ? (pair >> 4) : (pair & 15u));
    } else {
      v = e4m3_value(codes[((int64_t)g * c.p + off) * 32 + (ch & 31)]);
    }
    out[ch] = ldexpf(v, byte - 127);
  }
}

}  // namespace

hipError_t launch_append(const CacheGeom& c, uint8_t* kc, uint8_t* ks, uint8_t* vc, uint8_t* vs,
                         const uint16_t* k_new, const uint16_t* v_new, const int32_t* slots,
                         int n_tokens, hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  const AppendParams p = make_append_params(c, AppendArgs{kc, ks, vc, vs, k_new, v_new, slots, n_tokens});
  const int G = c.d / 32;
  const long long chunks = append_waves(c, n_tokens);  // waves per (head, tensor)
  const unsigned n_ht = (unsigned)c.hkv * (c.kv_shared ? 1u : 2u);
  const long long blocks = (n_ht & 3u) == 0 ? chunks * (long long)(n_ht / 4) : (chunks + 3) / 4 * (long long)n_ht;
  if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks);
  switch (G) {
    case 1: hipLaunchKernelGGL((append_kernel<1>), grid, dim3(256), 0, stream, p, n_ht); break;
    case 2: hipLaunchKernelGGL((append_kernel<2>), grid, dim3(256), 0, stream, p, n_ht); break;
    case 4: hipLaunchKernelGGL((append_kernel<4>), grid, dim3(256), 0, stream, p, n_ht); break;
    case 8: hipLaunchKernelGGL((append_kernel<8>), grid, dim3(256), 0, stream, p, n_ht); break;
    case 16: hipLaunchKernelGGL((append_kernel<16>), grid, dim3(256), 0, stream, p, n_ht); break;
    case 32: hipLaunchKernelGGL((append_kernel<32>), grid, dim3(256), 0, stream, p, n_ht); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dequant(const CacheGeom& c, const int32_t* slots, int n, float* k_out,
                          float* v_out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  DequantParams p;
  p.c = c;
  p.slots = slots;
  p.k_out = k_out;
  p.v_out = v_out;
  dim3 grid((unsigned)n, (unsigned)c.hkv, c.kv_shared ? 1u : 2u);
  hipLaunchKernelGGL(dequant_kernel, grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kvq
