// Kernel 2 (stand-alone form): G[r, s*d : (s+1)*d] = E_{n,k}[idx[r, s], :].
//
// This is the row read of the final form in section A2 of the deep-notes page on "Scaling
// Embeddings Outperforms Scaling Experts in Language Models": every position reads one
// d-wide row from each of the (N-1)K sub-tables, so the traffic is (N-1)K*d = D elements
// per position whatever the table sizes (section 4.1: lookup cost follows the token count).
// The projection kernel performs the same reads straight into LDS; this kernel writes them
// to HBM and is the bandwidth probe of the gather.
//
// Layout on MI355X: one grid row (blockIdx.y) per sub-table, so the table base is a
// wave-uniform scalar; each lane moves 16-byte vectors, consecutive lanes cover one table
// row (a 512-byte row is 32 lanes), and each lane keeps kUnroll independent rows in flight
// to cover HBM latency on random rows.
#include "kernels.h"

namespace ngram {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

struct GatherArgs {
  const char* E[NGRAM_MAX_SUBTABLES];
  uint32_t Vm1[NGRAM_MAX_SUBTABLES];  // V_{n,k} - 1, the largest valid index
  const int32_t* idx;                 // [nrows, S]
  char* G;                            // [nrows, D]
  int64_t nrows;
  int32_t S;
  uint32_t cpr;                       // 16-byte chunks per sub-table row
  uint32_t row_bytes;                 // d * esz
  uint32_t g_row_bytes;               // D * esz
};

__global__ __launch_bounds__(kThreads) void gather_kernel(const GatherArgs a) {
  const int s = blockIdx.y;
  const char* __restrict__ table = a.E[s];
  const uint32_t vmax = a.Vm1[s];
  // the host splits launches so that nrows * cpr < 2^30: 32-bit index math
  const uint32_t total = uint32_t(a.nrows) * a.cpr;
  const uint32_t base = blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  uint4 v[kUnroll];
  int64_t dst[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t item = base + u * kThreads;
    dst[u] = -1;
    if (item < total) {
      const uint32_t r = item / a.cpr;
      const uint32_t c = item - r * a.cpr;
      uint32_t id = uint32_t(a.idx[int64_t(r) * a.S + s]);
      id = id > vmax ? vmax : id;
      v[u] = *reinterpret_cast<const uint4*>(table + int64_t(id) * a.row_bytes + c * 16u);
      dst[u] = int64_t(r) * a.g_row_bytes + int64_t(s) * a.row_bytes + c * 16u;
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    if (dst[u] >= 0) *reinterpret_cast<uint4*>(a.G + dst[u]) = v[u];
}

}  // namespace

hipError_t launch_gather(const LayerDesc& L, const void* const* E, const int32_t* idx,
                         int64_t nrows, void* G, hipStream_t st) {
  GatherArgs a{};
  for (int s = 0; s < L.S; ++s) {
    a.E[s] = static_cast<const char*>(E[s]);
    a.Vm1[s] = L.V[s] - 1u;
  }
  a.S = L.S;
  a.row_bytes = uint32_t(L.d) * uint32_t(L.esz);
  a.cpr = a.row_bytes / 16u;
  a.g_row_bytes = uint32_t(L.D) * uint32_t(L.esz);
  const int64_t max_rows = (int64_t(1) << 30) / a.cpr;
  const int64_t per_block = int64_t(kThreads) * kUnroll;
  for (int64_t r0 = 0; r0 < nrows; r0 += max_rows) {
    const int64_t n = nrows - r0 < max_rows ? nrows - r0 : max_rows;
    a.idx = idx + r0 * L.S;
    a.G = static_cast<char*>(G) + r0 * int64_t(a.g_row_bytes);
    a.nrows = n;
    const unsigned bx = unsigned((n * a.cpr + per_block - 1) / per_block);
    hipLaunchKernelGGL(gather_kernel, dim3(bx, unsigned(L.S)), dim3(kThreads), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ngram
