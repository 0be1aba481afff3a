// The basic form of the N-gram embedding: section A2 (Eq. 1) of the deep-notes page on
// "Scaling Embeddings Outperforms Scaling Experts in Language Models":
//   out[r] = ( E_0[tok[r]] + sum_{n=2}^{N} E_n[idx[r, n-2]] ) / N,
// one table of full width D per order and no projection. Each output element is the sum of
// N table elements, so there is no contraction for the matrix cores: the kernel is a
// gather bound by HBM bandwidth, N rows read and one written per position
// ((N + 1) * D * esz bytes).
//
// Layout on MI355X: lane i of the grid owns 16-byte chunk i % cpr of output row i / cpr, so
// consecutive lanes cover consecutive chunks of one row and each of the N table rows is read
// as one contiguous piece (a 3072-wide bf16 row is 6 KB: 384 lanes, 6 waves). Every lane
// requests the row's token and ids together, then its N table pieces, before it adds (two
// memory round trips), keeps the sum in fp32 (E_0 first, then the tables in order), scales
// once and rounds once. Table loads stay cached (Zipf-distributed ids repeat
// within a batch); output stores are non-temporal, since nothing here reads them again.
// Rows whose token is outside [0, V0) are written as zeros, rows marked kSkipRow not at all,
// and the output row map places decode windows, as in the final form's epilogue.
#include "bf16.h"
#include "kernels.h"

namespace ngram {
namespace {

constexpr int kThreads = 256;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct SumArgs {
  const char* E[NGRAM_MAX_SUBTABLES];
  uint32_t Vm1[NGRAM_MAX_SUBTABLES];  // V_n - 1: indices are clamped to their table
  const char* E0;
  const int32_t* idx;                 // [nrows, S]
  const int32_t* tok;                 // [nrows]
  char* out;
  int64_t nrows;
  int32_t S, V0;
  int32_t cpr;                        // 16-byte chunks per table row: D * esz / 16
  int32_t row_bytes;                  // D * esz
  int32_t out_row_bytes;              // D * sizeof(output element)
  float inv;                          // output factor / N
  int32_t row_group, row_stride, row_off;
};

// Elements of one 16-byte chunk, added into acc[0 .. 16/sizeof(T)).
template <typename T> __device__ __forceinline__ void add_chunk(float* acc, const u32x4_t v);
template <> __device__ __forceinline__ void add_chunk<float>(float* acc, const u32x4_t v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] += __uint_as_float(v[i]);
}
template <> __device__ __forceinline__ void add_chunk<uint16_t>(float* acc, const u32x4_t v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] += bf16_to_f32(v[i] & 0xffffu);
    acc[2 * i + 1] += bf16_to_f32(v[i] >> 16);
  }
}

// SB: a bound on S (the orders after the first), so the row's ids sit in registers.
template <typename T, typename TO, int SB>
__global__ __launch_bounds__(kThreads) void basic_sum_kernel(const SumArgs a) {
  constexpr int kVec = 16 / sizeof(T);                  // elements per chunk
  const int64_t item = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (item >= a.nrows * a.cpr) return;
  const int64_t r = item / a.cpr;
  const int32_t c = int32_t(item - r * a.cpr);
  // the token and the ids first, all at once (the ids do not depend on the token), then
  // every table piece: two round trips to memory instead of three
  const int32_t tk = a.tok[r];
  const int32_t* id = a.idx + r * a.S;
  uint32_t ids[SB];
#pragma unroll
  for (int s = 0; s < SB; ++s) ids[s] = s < a.S ? uint32_t(id[s]) : 0u;
  if (tk == kSkipRow) return;
  float acc[kVec];
#pragma unroll
  for (int i = 0; i < kVec; ++i) acc[i] = 0.f;
  if (uint32_t(tk) < uint32_t(a.V0)) {
    const int64_t off = int64_t(c) * 16;
    u32x4_t piece[SB];
#pragma unroll
    for (int s = 0; s < SB; ++s) {
      const uint32_t x = ids[s] > a.Vm1[s] ? a.Vm1[s] : ids[s];
      if (s < a.S) piece[s] = *reinterpret_cast<const u32x4_t*>(a.E[s] + int64_t(x) * a.row_bytes + off);
    }
    add_chunk<T>(acc, *reinterpret_cast<const u32x4_t*>(a.E0 + int64_t(tk) * a.row_bytes + off));
#pragma unroll
    for (int s = 0; s < SB; ++s)
      if (s < a.S) add_chunk<T>(acc, piece[s]);
#pragma unroll
    for (int i = 0; i < kVec; ++i) acc[i] *= a.inv;
  }
  int64_t orow = r;
  if (a.row_group != 0)
    orow = (r / a.row_group) * a.row_stride + a.row_off + r % a.row_group;
  char* o = a.out + orow * a.out_row_bytes + int64_t(c) * kVec * int64_t(sizeof(TO));
  if constexpr (sizeof(TO) == 2) {                      // bf16 output: 8 values, 16 bytes
    u32x4_t w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = f32_to_bf16_rne(acc[2 * i]) | (f32_to_bf16_rne(acc[2 * i + 1]) << 16);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(o));
  } else {                                              // fp32 output: kVec / 4 vectors
#pragma unroll
    for (int q = 0; q < kVec / 4; ++q)
      __builtin_nontemporal_store(
          f32x4_t{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]},
          reinterpret_cast<f32x4_t*>(o) + q);
  }
}

// The basic form has K = 1: S = N - 1 <= NGRAM_MAX_ORDER - 1 orders after the first.
constexpr int kMaxBasicS = NGRAM_MAX_ORDER;

template <int SB>
hipError_t launch_sum(const LayerDesc& L, const SumArgs& a, dim3 grid, bool f32out,
                      hipStream_t st) {
  if (L.S > SB) return hipErrorInvalidValue;
  if (L.dtype == NGRAM_F32)
    hipLaunchKernelGGL((basic_sum_kernel<float, float, SB>), grid, dim3(kThreads), 0, st, a);
  else if (f32out)
    hipLaunchKernelGGL((basic_sum_kernel<uint16_t, float, SB>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((basic_sum_kernel<uint16_t, uint16_t, SB>), grid, dim3(kThreads), 0, st,
                       a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_basic(const LayerDesc& L, const void* E0, const void* const* E,
                        const int32_t* idx, const int32_t* tok, int64_t nrows, void* out,
                        bool f32out, const RowMap& map, hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  SumArgs a{};
  for (int s = 0; s < L.S; ++s) {
    a.E[s] = static_cast<const char*>(E[s]);
    a.Vm1[s] = L.V[s] - 1u;
  }
  a.E0 = static_cast<const char*>(E0);
  a.idx = idx;
  a.tok = tok;
  a.out = static_cast<char*>(out);
  a.nrows = nrows;
  a.S = L.S;
  a.V0 = L.V0;
  a.row_bytes = L.D * L.esz;
  a.cpr = a.row_bytes / 16;
  a.out_row_bytes = L.D * (f32out ? 4 : L.esz);
  a.inv = L.scale / float(L.S + 1);
  a.row_group = map.group;
  a.row_stride = map.stride;
  a.row_off = map.off;
  const int64_t blocks = (nrows * a.cpr + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid{unsigned(blocks)};
  if (L.S <= 4) return launch_sum<4>(L, a, grid, f32out, st);
  return launch_sum<kMaxBasicS>(L, a, grid, f32out, st);
}

}  // namespace ngram
