// Kernel 2 alone: the row reads G[r, s*d : (s+1)*d] = E_{n,k}[idx[r, s], :].
//
// This is the row read of the final form in section A2 of the deep-notes page on "Scaling
// Embeddings Outperforms Scaling Experts in Language Models": every position reads one
// d-wide row from each of the (N-1)K sub-tables, so the traffic is (N-1)K*d = D elements
// per position whatever the table sizes (section 4.1: lookup cost follows the token count).
// The projection kernel performs these reads straight into LDS. Two stand-alone forms:
// gather_kernel writes G to HBM (ngram_embed_gather), and gather_lds_kernel lands the rows
// in LDS with the projection's loader and keeps one checksum per row
// (ngram_embed_gather_checksum), the bandwidth probe of the gather as the path runs it.
//
// Layout of the HBM form on MI355X: idx [rows, S] and G [rows, S*d] list the (row, sub-table) pairs in the
// same order, so G is a flat array of pair segments: 16-byte chunk `item` of G is chunk
// item % cpr of pair item / cpr. Consecutive lanes take consecutive chunks: every table row
// is read as one contiguous piece and every write is fully sequential. Stores are
// non-temporal (G is not re-read here); loads stay cached, since with Zipf-distributed ids
// many n-grams repeat within a batch. Each lane keeps kUnroll chunks in flight. These
// choices measured best on the 30B-parameter layer with Zipf(1.1) ids.
#include <algorithm>

#include "kernels.h"
#include "lds_dma.h"

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

// ------------------------------------------------------------------ gather into LDS
// The gather as the projection performs it: sub-table rows from HBM straight into LDS with
// the same 16-byte-per-lane LDS loads (global_load_lds_dwordx4), nothing written back to
// HBM. What lands is reduced in place to one order-sensitive checksum per gathered row,
//   sum[r] = sum_k w_k * (2k + 1)  (mod 2^32)
// over the 32-bit words w_k of the row r = [E_s[idx[r, s]] for s = 0..S-1] (the row that
// ngram_embed_gather writes), so a test can check every landed byte against the tables and
// a benchmark sees HBM -> LDS traffic alone (4 bytes written per row).
// The rate is set by the bytes each CU keeps in flight, so the work between a wave's batches
// is kept short: every wave owns kWaveKB KB of LDS and takes batches of whole rows that fill
// it (3 rows of 6 KB for 12 sub-tables of 512 bytes), issues all of a batch's loads, then the
// indices of its next batch, and only then waits. With the loads per row a compile-time
// count (NI: 1, 2, 4 or 6 for the shapes measured), each lane's table base, clamp and chunk
// offset per load are fixed for the whole kernel, a row's index shuffles go out together
// before its loads, and the row sums are reduced with DPP moves rather than through LDS.
constexpr int kLdsWaves = 8;
constexpr int kWaveKB = 19;          // 8 waves x 19 KB, and the sub-table table: 160 KB of LDS

struct GatherLdsArgs {
  const char* E[NGRAM_MAX_SUBTABLES];
  uint32_t Vm1[NGRAM_MAX_SUBTABLES];  // V_{n,k} - 1, the largest valid index
  const int32_t* idx;                 // [rows, S]
  uint32_t* sums;                     // [rows]
  int64_t nrows;
  uint32_t S;
  uint32_t cpr;                       // 16-byte chunks per sub-table row
  uint32_t row_bytes;                 // d * esz
  uint32_t ni;                        // 1 KB wave loads per gathered row: ceil(S * cpr / 64)
  uint32_t rpb;                       // rows per batch (rpb * ni <= kWaveKB, rpb * S <= 64);
                                      // 0: rows longer than the buffer, taken in pieces
};

// Sum over the wave's 64 lanes, returned in every lane: DPP within rows of 16 lanes
// (quad swaps, then the half-row and row mirrors), then the four row totals.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x4E, 0xF, 0xF, false));   // [2,3,0,1]
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x141, 0xF, 0xF, false));  // half mirror
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x140, 0xF, 0xF, false));  // row mirror
  return uint32_t(__builtin_amdgcn_readlane(int(v), 0)) +
         uint32_t(__builtin_amdgcn_readlane(int(v), 16)) +
         uint32_t(__builtin_amdgcn_readlane(int(v), 32)) +
         uint32_t(__builtin_amdgcn_readlane(int(v), 48));
}

// Checksum terms of 16-byte chunk g of a gathered row (its words 4g .. 4g+3).
__device__ __forceinline__ uint32_t chunk_terms(const u32x4_t v, uint32_t g) {
  const uint32_t k = 8u * g + 1u;                    // 2 * (4g) + 1
  return v.x * k + v.y * (k + 2u) + v.z * (k + 4u) + v.w * (k + 6u);
}

// NI > 0: every gathered row takes exactly NI wave loads (batches of rpb rows); NI == 0:
// the general form (any count; rows longer than the buffer go in pieces).
template <int NI>
__global__ __launch_bounds__(kLdsWaves * 64) void gather_lds_kernel(const GatherLdsArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsWaves * kWaveKB * 1024];
  // each sub-table's base and largest index, read per lane from LDS: per-lane reads of the
  // kernel arguments would be vector loads, and the compiler would wait for every load in
  // flight (the LDS loads included) before each address they feed
  __shared__ const char* sE[NGRAM_MAX_SUBTABLES];
  __shared__ uint32_t sVm1[NGRAM_MAX_SUBTABLES];
  if (threadIdx.x < a.S) {
    sE[threadIdx.x] = a.E[threadIdx.x];
    sVm1[threadIdx.x] = a.Vm1[threadIdx.x];
  }
  __syncthreads();
  const uint32_t lane = threadIdx.x & 63u;
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const uint32_t wbuf = uint32_t(w) * kWaveKB * 1024u;     // this wave's LDS, byte offset
  const uint32_t lds0 = lds_address(lds) + wbuf;
  const int64_t nwaves = int64_t(gridDim.x) * kLdsWaves;
  const int64_t wid = int64_t(blockIdx.x) * kLdsWaves + w;
  const uint32_t per_row = a.S * a.cpr;                    // 16-byte chunks of a gathered row
  // Load j of a row: this lane's chunk g = 64 j + lane is chunk g % cpr of sub-table g / cpr;
  // the index of batch row rr and sub-table s sits in lane rr * S + s of the batch's indices.
  auto slot_of = [&](uint32_t j, uint32_t* s, const char** base, uint32_t* vm) __attribute__((always_inline)) {
    const uint32_t g = j * 64u + lane;
    *s = min(g / a.cpr, a.S - 1u);
    *base = sE[*s] + (g - *s * a.cpr) * 16u;
    *vm = sVm1[*s];
    return g < per_row;
  };
  if constexpr (NI > 0) {
    uint32_t ls[NI], lvm[NI];
    const char* lbase[NI];
    bool lok[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) lok[j] = slot_of(j, &ls[j], &lbase[j], &lvm[j]);
    const int64_t nbatch = (a.nrows + a.rpb - 1) / a.rpb;
    auto rows_of = [&](int64_t b) __attribute__((always_inline)) {
      return b < nbatch ? uint32_t(min(int64_t(a.rpb), a.nrows - b * a.rpb)) : 0u;
    };
    auto batch_idx = [&](int64_t b) __attribute__((always_inline)) {
      return lane < rows_of(b) * a.S ? a.idx[b * a.rpb * a.S + lane] : 0;
    };
    int32_t myidx = batch_idx(wid);
    for (int64_t b = wid; b < nbatch; b += nwaves) {
      // The batch's indices have arrived (nothing of the wave is in flight here). Said with
      // the builtin, which the compiler's wait placement understands (it cannot see into
      // asm): otherwise it waits for them before every load below, draining the loads in
      // flight each time. 0xF70: vmcnt(0), the other counters unconstrained.
      __builtin_amdgcn_s_waitcnt(0xF70);
      const uint32_t nr = rows_of(b);
      for (uint32_t rr = 0; rr < nr; ++rr) {
        uint32_t id[NI];
#pragma unroll
        for (int j = 0; j < NI; ++j) id[j] = uint32_t(__shfl(myidx, int(rr * a.S + ls[j]), 64));
#pragma unroll
        for (int j = 0; j < NI; ++j)
          if (lok[j])
            dma16(lbase[j] + int64_t(min(id[j], lvm[j])) * a.row_bytes,
                  lds0 + (rr * NI + j) * 1024u);
      }
      myidx = batch_idx(b + nwaves);                       // the next batch's indices
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      for (uint32_t rr = 0; rr < nr; ++rr) {
        u32x4_t v[NI];
#pragma unroll
        for (int j = 0; j < NI; ++j)
          v[j] = *reinterpret_cast<const u32x4_t*>(lds + wbuf + (rr * NI + j) * 1024u + lane * 16u);
        uint32_t part = 0;
#pragma unroll
        for (int j = 0; j < NI; ++j)
          if (lok[j]) part += chunk_terms(v[j], uint32_t(j) * 64u + lane);
        part = wave_sum(part);
        if (lane == 0) a.sums[b * a.rpb + rr] = part;
      }
      // every lane's LDS reads are done before the next batch's loads overwrite the buffer
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  } else {
    // any load count: one row at a time, up to kWaveKB loads per piece
    for (int64_t r = wid; r < a.nrows; r += nwaves) {
      const int32_t myidx = lane < a.S ? a.idx[r * a.S + lane] : 0;
      __builtin_amdgcn_s_waitcnt(0xF70);   // as above: the indices first, then only the loads
      uint32_t part = 0;
      for (uint32_t j0 = 0; j0 < a.ni; j0 += kWaveKB) {
        const uint32_t nj = min(a.ni - j0, uint32_t(kWaveKB));
        for (uint32_t j = 0; j < nj; ++j) {
          uint32_t s, vm;
          const char* base;
          const bool ok = slot_of(j0 + j, &s, &base, &vm);
          const uint32_t id = min(uint32_t(__shfl(myidx, int(s), 64)), vm);
          if (ok) dma16(base + int64_t(id) * a.row_bytes, lds0 + j * 1024u);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        for (uint32_t j = 0; j < nj; ++j) {
          const uint32_t g = (j0 + j) * 64u + lane;
          if (g < per_row)
            part += chunk_terms(*reinterpret_cast<const u32x4_t*>(lds + wbuf + j * 1024u +
                                                                   lane * 16u), g);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
      part = wave_sum(part);
      if (lane == 0) a.sums[r] = part;
    }
  }
}

}  // namespace

hipError_t launch_gather_lds(const LayerDesc& L, const void* const* E, const int32_t* idx,
                             int64_t nrows, uint32_t* sums, hipStream_t st) {
  if (nrows <= 0 || L.S <= 0) return hipSuccess;
  GatherLdsArgs a{};
  for (int s = 0; s < L.S; ++s) {
    a.E[s] = static_cast<const char*>(E[s]);
    a.Vm1[s] = L.V[s] - 1u;
  }
  a.idx = idx;
  a.sums = sums;
  a.nrows = nrows;
  a.S = uint32_t(L.S);
  a.row_bytes = uint32_t(L.d) * uint32_t(L.esz);
  a.cpr = a.row_bytes / 16u;
  a.ni = (a.S * a.cpr + 63u) / 64u;
  // batches of whole rows that fill the wave's buffer (their indices in <= 64 lanes)
  a.rpb = std::min(uint32_t(kWaveKB) / a.ni, 64u / a.S);
  const int64_t units = a.rpb > 0 ? (nrows + a.rpb - 1) / a.rpb : nrows;
  // one block per CU (the whole LDS), its waves striding over the batches
  const dim3 grid(unsigned(std::min<int64_t>((units + kLdsWaves - 1) / kLdsWaves, 256)));
  const dim3 block(kLdsWaves * 64);
  if (a.rpb > 0 && a.ni == 6) hipLaunchKernelGGL(gather_lds_kernel<6>, grid, block, 0, st, a);
  else if (a.rpb > 0 && a.ni == 4) hipLaunchKernelGGL(gather_lds_kernel<4>, grid, block, 0, st, a);
  else if (a.rpb > 0 && a.ni == 2) hipLaunchKernelGGL(gather_lds_kernel<2>, grid, block, 0, st, a);
  else if (a.rpb > 0 && a.ni == 1) hipLaunchKernelGGL(gather_lds_kernel<1>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(gather_lds_kernel<0>, grid, block, 0, st, a);
  return hipGetLastError();
}

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
