// Kernel 2 (stand-alone form): G[r, s*d : (s+1)*d] = E_{n,k}[idx[r, s], :].
//
// This is the row read of the final form in section A2 of the deep-notes page on "Scaling
// Embeddings Outperforms Scaling Experts in Language Models": every position reads one
// d-wide row from each of the (N-1)K sub-tables, so the traffic is (N-1)K*d = D elements
// per position whatever the table sizes (section 4.1: lookup cost follows the token count).
// The projection kernel performs the same reads straight into LDS; this kernel writes them
// to HBM and is the bandwidth probe of the gather.
//
// Layout on MI355X: idx [rows, S] and G [rows, S*d] list the (row, sub-table) pairs in the
// same order, so G is a flat array of pair segments: 16-byte chunk `item` of G is chunk
// item % cpr of pair item / cpr. Consecutive lanes take consecutive chunks: every table row
// is read as one contiguous piece and every write is fully sequential. Stores are
// non-temporal (G is not re-read here); loads stay cached, since with Zipf-distributed ids
// many n-grams repeat within a batch. Each lane keeps kUnroll chunks in flight. These
// choices measured best on the 30B-parameter layer with Zipf(1.1) ids.
#include "kernels.h"

namespace ngram {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 2;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct GatherArgs {
  const char* E[NGRAM_MAX_SUBTABLES];
  uint32_t Vm1[NGRAM_MAX_SUBTABLES];  // V_{n,k} - 1, the largest valid index
  const int32_t* idx;                 // [rows, S]
  char* G;                            // [rows, S * d]
  uint32_t total;                     // 16-byte chunks in this launch: rows * S * cpr
  uint32_t S;
  uint32_t cpr;                       // 16-byte chunks per sub-table row (d * esz / 16)
  uint32_t row_bytes;                 // d * esz
};

__global__ __launch_bounds__(kThreads) void gather_kernel(const GatherArgs a) {
  const uint32_t base = blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  u32x4_t v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t item = base + u * kThreads;
    if (item < a.total) {
      const uint32_t p = item / a.cpr;                 // (row, sub-table) pair
      const uint32_t c = item - p * a.cpr;             // chunk within the row
      const uint32_t s = p % a.S;
      uint32_t id = uint32_t(a.idx[p]);
      id = id > a.Vm1[s] ? a.Vm1[s] : id;
      v[u] = *reinterpret_cast<const u32x4_t*>(a.E[s] + int64_t(id) * a.row_bytes + c * 16u);
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t item = base + u * kThreads;
    if (item < a.total)
      __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4_t*>(a.G + int64_t(item) * 16));
  }
}

}  // namespace

hipError_t launch_gather(const LayerDesc& L, const void* const* E, const int32_t* idx,
                         int64_t nrows, void* G, hipStream_t st) {
  GatherArgs a{};
  for (int s = 0; s < L.S; ++s) {
    a.E[s] = static_cast<const char*>(E[s]);
    a.Vm1[s] = L.V[s] - 1u;
  }
  a.S = uint32_t(L.S);
  a.row_bytes = uint32_t(L.d) * uint32_t(L.esz);
  a.cpr = a.row_bytes / 16u;
  // 32-bit chunk numbering: launches of at most 2^30 chunks, whole rows each
  const int64_t chunks_per_row = int64_t(L.S) * a.cpr;
  const int64_t max_rows = (int64_t(1) << 30) / chunks_per_row;
  const int64_t per_block = int64_t(kThreads) * kUnroll;
  for (int64_t r0 = 0; r0 < nrows; r0 += max_rows) {
    const int64_t n = nrows - r0 < max_rows ? nrows - r0 : max_rows;
    a.idx = idx + r0 * L.S;
    a.G = static_cast<char*>(G) + r0 * chunks_per_row * 16;
    a.total = uint32_t(n * chunks_per_row);
    const unsigned blocks = unsigned((int64_t(a.total) + per_block - 1) / per_block);
    hipLaunchKernelGGL(gather_kernel, dim3(blocks), dim3(kThreads), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ngram
