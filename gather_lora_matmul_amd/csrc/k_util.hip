// Pool maintenance kernels (NaN poisoning, page scatter of an upload) and the
// verification kernels that expose the in-kernel page-table resolution.
#include "kcommon.h"

namespace lora {

__global__ void k_fill_words(uint32_t* __restrict__ p, int64_t nwords, uint32_t word) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nwords;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = word;
}

// Page j of the list gets the 32-bit pattern everywhere.
__global__ void k_fill_pages(char* __restrict__ pages, int64_t page_bytes,
                             const int32_t* __restrict__ ids, uint32_t word) {
  uint32_t* dst = reinterpret_cast<uint32_t*>(pages + (int64_t)ids[blockIdx.x] * page_bytes);
  for (int64_t i = threadIdx.x; i < page_bytes / 4; i += blockDim.x) dst[i] = word;
}

// Page j of the staging buffer goes to pool page ids[j] (16-byte copies).
__global__ void k_scatter_pages(char* __restrict__ pages, int64_t page_bytes,
                                const char* __restrict__ staging, const int32_t* __restrict__ ids) {
  const int64_t j = blockIdx.x;
  const uint4* src = reinterpret_cast<const uint4*>(staging + j * page_bytes);
  uint4* dst = reinterpret_cast<uint4*>(pages + (int64_t)ids[j] * page_bytes);
  for (int64_t i = threadIdx.x; i < page_bytes / 16; i += blockDim.x) dst[i] = src[i];
}

static uint32_t pattern_word(uint32_t pattern, int elt) {
  if (elt == 1) return (pattern & 0xffu) * 0x01010101u;
  return elt == 4 ? pattern : (pattern & 0xffffu) | (pattern << 16);
}

hipError_t launch_fill_all(char* pages, int64_t bytes, uint32_t pattern, int elt, hipStream_t s) {
  const int64_t nwords = bytes / 4;
  const int64_t blocks = std::min<int64_t>((nwords + 255) / 256, 1 << 16);
  hipLaunchKernelGGL(k_fill_words, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, s,
                     reinterpret_cast<uint32_t*>(pages), nwords, pattern_word(pattern, elt));
  return hipGetLastError();
}

hipError_t launch_fill_pages(char* pages, int64_t page_bytes, const int32_t* ids_dev, int64_t n,
                             uint32_t pattern, int elt, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_pages, dim3((unsigned)n), dim3(256), 0, s, pages, page_bytes, ids_dev,
                     pattern_word(pattern, elt));
  return hipGetLastError();
}

hipError_t launch_scatter_pages(char* pages, int64_t page_bytes, const char* staging,
                                const int32_t* ids_dev, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_scatter_pages, dim3((unsigned)n), dim3(256), 0, s, pages, page_bytes,
                     staging, ids_dev);
  return hipGetLastError();
}

// ---- resolution exposed for bit-exact checks --------------------------------
// Block per token: A offsets for k < max_rank (all page chunks), B row offsets.
__global__ void k_debug_resolve(PoolView pv, IoDesc io, int max_rank, int elt,
                                const int32_t* __restrict__ ids, int64_t* __restrict__ a_off,
                                int64_t* __restrict__ b_off) {
  const int i = blockIdx.x;
  const int a = ids[i];
  DevEntry e;
  e.rank = 0;
  if (adapter_in_table(pv, a)) e = pv.entries[io.slice * pv.max_adapters + a];
  const int na = max_rank * io.npa;
  for (int idx = threadIdx.x; idx < na; idx += blockDim.x) {
    const int k = idx / io.npa;
    const int c = idx - k * io.npa;
    a_off[(int64_t)i * na + idx] = k < e.rank ? a_offset(pv, e, io.npa, elt, k, c * pv.P) : -1;
  }
  for (int m = threadIdx.x; m < io.d_out; m += blockDim.x)
    b_off[(int64_t)i * io.d_out + m] = e.rank > 0 ? b_offset(pv, e, elt, m) : -1;
}

// Dense copy of one adapter slice, element by element through the resolver.
__global__ void k_debug_gather(PoolView pv, IoDesc io, int elt, int adapter, int rank,
                               char* __restrict__ A, char* __restrict__ B) {
  const DevEntry e = pv.entries[io.slice * pv.max_adapters + adapter];
  const int64_t na = (int64_t)rank * io.d_in;
  const int64_t nb = (int64_t)io.d_out * rank;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < na + nb; idx += stride) {
    const char* src;
    char* dst;
    if (idx < na) {
      const int k = (int)(idx / io.d_in);
      const int j = (int)(idx - (int64_t)k * io.d_in);
      src = pv.pages + a_offset(pv, e, io.npa, elt, k, j);
      dst = A + idx * elt;
    } else {
      const int64_t t = idx - na;
      const int m = (int)(t / rank);
      const int k = (int)(t - (int64_t)m * rank);
      src = pv.pages + b_offset(pv, e, elt, m) + (int64_t)k * elt;
      dst = B + t * elt;
    }
    if (elt == 4)
      *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(src);
    else if (elt == 2)
      *reinterpret_cast<uint16_t*>(dst) = *reinterpret_cast<const uint16_t*>(src);
    else
      *dst = *src;
  }
}

// Stored elements -> fp32 through the compute kernels' own decoder (unpack16),
// one 16-byte chunk per thread.
template <typename T>
__global__ void k_debug_decode(const char* __restrict__ src, int64_t nchunks, float* __restrict__ dst) {
  const int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (c >= nchunks) return;
  float f[ET<T>::E];
  unpack16<T>(ld16(src + c * 16), f);
#pragma unroll
  for (int e = 0; e < ET<T>::E; ++e) dst[c * ET<T>::E + e] = f[e];
}

hipError_t launch_debug_decode(int dtype, const void* src, int64_t n, float* dst, hipStream_t s) {
  const int elt = dtype == LORA_F32 ? 4 : (dtype == LORA_FP8_E4M3 ? 1 : 2);
  const int64_t nchunks = n * elt / 16;
  if (nchunks <= 0) return hipSuccess;
  const dim3 grid((unsigned)((nchunks + 255) / 256));
  const char* p = reinterpret_cast<const char*>(src);
  switch (dtype) {
    case LORA_F32: hipLaunchKernelGGL(k_debug_decode<float>, grid, dim3(256), 0, s, p, nchunks, dst); break;
    case LORA_F16: hipLaunchKernelGGL(k_debug_decode<f16_t>, grid, dim3(256), 0, s, p, nchunks, dst); break;
    case LORA_BF16: hipLaunchKernelGGL(k_debug_decode<bf16_t>, grid, dim3(256), 0, s, p, nchunks, dst); break;
    default: hipLaunchKernelGGL(k_debug_decode<fp8_t>, grid, dim3(256), 0, s, p, nchunks, dst); break;
  }
  return hipGetLastError();
}

hipError_t launch_debug_resolve(const PoolView& pv, const IoDesc& io, int32_t max_rank, int elt,
                                const int32_t* ids, int32_t n, int64_t* a_off, int64_t* b_off,
                                hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_debug_resolve, dim3(n), dim3(256), 0, s, pv, io, max_rank, elt, ids, a_off,
                     b_off);
  return hipGetLastError();
}

hipError_t launch_debug_gather(int elt, const PoolView& pv, const IoDesc& io, int32_t adapter,
                               int32_t rank, void* A, void* B, hipStream_t s) {
  hipLaunchKernelGGL(k_debug_gather, dim3(1024), dim3(256), 0, s, pv, io, elt, adapter, rank,
                     reinterpret_cast<char*>(A), reinterpret_cast<char*>(B));
  return hipGetLastError();
}

}  // namespace lora
