// Expert permutation of the routing slots (histogram, prefix scan, stable
// rank) and the dynamic FP8 quantisation of activations gathered into expert
// order.
//
// Slots are s = t*k + j.  Rows of one expert keep ascending slot (hence
// token) order, so the result is deterministic: no atomic decides a row.
#include "moe_internal.h"
#include "fp8_rows.h"

namespace moe {

// ---------------------------------------------------------------------------
// Pass 1: per-block expert histogram of kPermBlock slots (LDS atomics only
// count; they decide no position).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) perm_count_kernel(const int32_t* __restrict__ ids,
                                                          int32_t* __restrict__ block_counts,
                                                          int N, int E) {
    __shared__ int cnt[512];
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    const int s = blockIdx.x * kPermBlock + threadIdx.x;
    if (s < N) {
        const int e = ids[s];
        if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);   // out-of-range ids are dropped
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) block_counts[(size_t)blockIdx.x * E + e] = cnt[e];
}

// ---------------------------------------------------------------------------
// Pass 2 (one workgroup): for each expert, the exclusive prefix over blocks
// (block_base), then the exclusive prefix over experts of the totals
// (offsets[0..E], offsets[E] = N).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(512) perm_scan_kernel(const int32_t* __restrict__ block_counts,
                                                        int32_t* __restrict__ block_base,
                                                        int32_t* __restrict__ offsets, int nblk, int E) {
    __shared__ int tot[512];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        for (int b = 0; b < nblk; ++b) {
            const int c = block_counts[(size_t)b * E + e];
            block_base[(size_t)b * E + e] = run;
            run += c;
        }
    }
    tot[e] = (e < E) ? run : 0;
    __syncthreads();
    // Hillis-Steele inclusive scan over 512 entries
    for (int d = 1; d < 512; d <<= 1) {
        const int v = (e >= d) ? tot[e - d] : 0;
        __syncthreads();
        tot[e] += v;
        __syncthreads();
    }
    if (e < E) offsets[e] = tot[e] - run;
    if (e == E - 1) offsets[E] = tot[e];
}

// ---------------------------------------------------------------------------
// Pass 3: row of every slot = offsets[e] + block_base[b][e] + (slots of e in
// earlier waves of this block) + (slots of e in earlier lanes of this wave).
// The in-wave match mask is built from one ballot per bit of the expert id.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) perm_scatter_kernel(const int32_t* __restrict__ ids,
                                                            const int32_t* __restrict__ block_base,
                                                            const int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ sorted_token,
                                                            int32_t* __restrict__ row_of_slot,
                                                            int N, int E, int k) {
    __shared__ int wcnt[16][512];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < 16 * 512; i += blockDim.x) (&wcnt[0][0])[i] = 0;
    const int s = blockIdx.x * kPermBlock + threadIdx.x;
    const int id = s < N ? ids[s] : -1;
    const bool valid = (unsigned)id < (unsigned)E;
    const int e = valid ? id : 1023;   // 1023 never equals a real id (E <= 512)

    unsigned long long m = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 10; ++bit) {
        const unsigned long long b = __ballot((e >> bit) & 1);
        m &= ((e >> bit) & 1) ? b : ~b;
    }
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(m & lt);
    __syncthreads();   // wcnt cleared
    if (valid && rank == 0) wcnt[wave][e] = __popcll(m);
    __syncthreads();
    if (!valid) {
        if (s < N) row_of_slot[s] = -1;   // an out-of-range id gets no row
        return;
    }
    int pre = 0;
    for (int w = 0; w < wave; ++w) pre += wcnt[w][e];
    const int row = offsets[e] + block_base[(size_t)blockIdx.x * E + e] + pre + rank;
    row_of_slot[s] = row;
    sorted_token[row] = s / k;
}

// ---------------------------------------------------------------------------
// All of the permutation for at most kPermBlock slots (decode), plus the
// tiled GEMMs' tile plan, in one workgroup: expert histogram, the two
// exclusive scans (rows and m-tiles), the stable in-block rank of every slot
// (the ballot match of perm_scatter_kernel) and the per-tile descriptors
// (max_tiles of them; 0 when the streaming GEMMs run, which need none).
// One launch instead of four.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kPermBlock) perm_small_kernel(const int32_t* __restrict__ ids,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ sorted_token,
                                                                int32_t* __restrict__ row_of_slot,
                                                                int32_t* __restrict__ tile_start,
                                                                int4* __restrict__ tile_info,
                                                                int N, int E, int k, int rpt, int max_tiles) {
    __shared__ int cnt[512];
    __shared__ int2 scan[512];          // (rows, tiles) inclusive prefix
    __shared__ int off[513], tst[513];
    __shared__ int wcnt[kPermBlock / 64][512];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < 512; i += kPermBlock) cnt[i] = 0;
    for (int i = tid; i < (kPermBlock / 64) * 512; i += kPermBlock) (&wcnt[0][0])[i] = 0;
    __syncthreads();
    const int id = tid < N ? ids[tid] : -1;
    const bool valid = (unsigned)id < (unsigned)E;
    const int e = valid ? id : 1023;    // 1023 never equals a real id (E <= 512)
    if (valid) atomicAdd(&cnt[e], 1);   // counts only; no position depends on the order
    __syncthreads();
    // inclusive scan of (rows, tiles) over 512 experts: Hillis-Steele on threads 0..511
    int n = 0, nt = 0;
    if (tid < 512) {
        n = tid < E ? cnt[tid] : 0;
        nt = (n + rpt - 1) / rpt;
        scan[tid] = int2{n, nt};
    }
    __syncthreads();
    for (int d = 1; d < 512; d <<= 1) {
        int2 v = int2{0, 0};
        if (tid < 512 && tid >= d) v = scan[tid - d];
        __syncthreads();
        if (tid < 512) { scan[tid].x += v.x; scan[tid].y += v.y; }
        __syncthreads();
    }
    if (tid < E) {
        off[tid] = scan[tid].x - n;
        tst[tid] = scan[tid].y - nt;
        offsets[tid] = scan[tid].x - n;
        tile_start[tid] = scan[tid].y - nt;
    }
    if (tid == E - 1) {
        off[E] = scan[tid].x; tst[E] = scan[tid].y;
        offsets[E] = scan[tid].x; tile_start[E] = scan[tid].y;
    }
    // stable rank of each slot among the slots of its expert
    unsigned long long m = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 10; ++bit) {
        const unsigned long long b = __ballot((e >> bit) & 1);
        m &= ((e >> bit) & 1) ? b : ~b;
    }
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(m & lt);
    if (valid && rank == 0) wcnt[wave][e] = __popcll(m);
    __syncthreads();
    if (tid < N) {
        if (valid) {
            int pre = 0;
            for (int w = 0; w < wave; ++w) pre += wcnt[w][e];
            const int row = off[e] + pre + rank;
            row_of_slot[tid] = row;
            sorted_token[row] = tid / k;
        } else {
            row_of_slot[tid] = -1;   // an out-of-range id gets no row
        }
    }
    // per-tile descriptors {expert, first row, rows}; expert -1 past the last tile
    const int ntiles = tst[E];
    for (int t = tid; t < max_tiles; t += kPermBlock) {
        int4 info = {-1, 0, 0, 0};
        if (t < ntiles) {
            int lo = 0, hi = E - 1;   // largest expert whose first tile is <= t
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (tst[mid] <= t) lo = mid; else hi = mid - 1;
            }
            const int row0 = off[lo] + (t - tst[lo]) * rpt;
            info = int4{lo, row0, min(rpt, off[lo + 1] - row0), 0};
        }
        tile_info[t] = info;
    }
}

hipError_t launch_perm_small(const int32_t* ids, int32_t* offsets, int32_t* sorted_token, int32_t* row_of_slot,
                             int32_t* tile_start, int4* tile_info, int64_t N, int E, int k, int rows_per_tile,
                             int max_tiles, hipStream_t stream) {
    hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(kPermBlock), 0, stream, ids, offsets, sorted_token,
                       row_of_slot, tile_start, tile_info, (int)N, E, k, rows_per_tile, max_tiles);
    return hipGetLastError();
}

hipError_t launch_perm_count(const int32_t* ids, int32_t* block_counts, int64_t N, int E,
                             hipStream_t stream) {
    const int nblk = (int)((N + kPermBlock - 1) / kPermBlock);
    hipLaunchKernelGGL(perm_count_kernel, dim3(nblk), dim3(kPermBlock), 0, stream, ids, block_counts, (int)N, E);
    return hipGetLastError();
}

hipError_t launch_perm_scan(const int32_t* block_counts, int32_t* block_base, int32_t* offsets, int64_t N,
                            int E, hipStream_t stream) {
    const int nblk = (int)((N + kPermBlock - 1) / kPermBlock);
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(512), 0, stream, block_counts, block_base, offsets, nblk, E);
    return hipGetLastError();
}

hipError_t launch_perm_scatter(const int32_t* ids, const int32_t* block_base, const int32_t* offsets,
                               int32_t* sorted_token, int32_t* row_of_slot, int64_t N, int E, int k,
                               hipStream_t stream) {
    const int nblk = (int)((N + kPermBlock - 1) / kPermBlock);
    hipLaunchKernelGGL(perm_scatter_kernel, dim3(nblk), dim3(kPermBlock), 0, stream, ids, block_base, offsets,
                       sorted_token, row_of_slot, (int)N, E, k);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Quantise + gather: row r of the output is FP8(x[sorted_token[r]]), or
// FP8(x[r]) without sorted_token (the gather then happens in GEMM-1).  The
// row quantiser itself is in fp8_rows.h.
// ---------------------------------------------------------------------------
template <bool F32S>
__global__ void __launch_bounds__(256) quant_gather_kernel(const uint16_t* __restrict__ x,
                                                           const int32_t* __restrict__ sorted_token,
                                                           uint8_t* __restrict__ xq, void* __restrict__ xs,
                                                           int N, int H, int T) {
    for (int r = blockIdx.x; r < N; r += gridDim.x) {
        // (no sorted_token: quantise the tokens in their own order)
        const int t = sorted_token ? min(max(sorted_token[r], 0), T - 1) : r;   // rows left unfilled by invalid ids stay in bounds
        quantise_row<F32S>(x + (size_t)t * H, xq, xs, r, H);
    }
}

hipError_t launch_quant_gather(const uint16_t* x, const int32_t* sorted_token, uint8_t* xq, void* xs,
                               int64_t N, int H, int64_t T, int f32_scales, hipStream_t stream) {
    const int grid = (int)(N < 65536 ? N : 65536);
    if (f32_scales)
        hipLaunchKernelGGL(quant_gather_kernel<true>, dim3(grid), dim3(256), 0, stream, x, sorted_token, xq, xs,
                           (int)N, H, (int)T);
    else
        hipLaunchKernelGGL(quant_gather_kernel<false>, dim3(grid), dim3(256), 0, stream, x, sorted_token, xq, xs,
                           (int)N, H, (int)T);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Tile plan of the grouped GEMMs: expert e owns m-tiles
// [tile_start[e], tile_start[e+1]) of rows_per_tile rows each.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(512) tile_plan_kernel(const int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ tile_start, int4* __restrict__ tile_info,
                                                        int E, int rpt, int max_tiles) {
    __shared__ int tot[512];
    __shared__ int start[513];
    __shared__ int off[513];
    const int e = threadIdx.x;
    const int o0 = (e < E) ? offsets[e] : 0, o1 = (e < E) ? offsets[e + 1] : 0;
    const int n = (e < E) ? (o1 - o0 + rpt - 1) / rpt : 0;
    tot[e] = n;
    __syncthreads();
    for (int d = 1; d < 512; d <<= 1) {
        const int v = (e >= d) ? tot[e - d] : 0;
        __syncthreads();
        tot[e] += v;
        __syncthreads();
    }
    if (e < E) { start[e] = tot[e] - n; off[e] = o0; tile_start[e] = tot[e] - n; }
    if (e == E - 1) { start[E] = tot[e]; off[E] = o1; tile_start[E] = tot[e]; }
    __syncthreads();
    const int ntiles = start[E];
    for (int t = e; t < max_tiles; t += 512) {
        int4 info = {-1, 0, 0, 0};
        if (t < ntiles) {
            int lo = 0, hi = E - 1;   // largest expert whose first tile is <= t
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (start[mid] <= t) lo = mid; else hi = mid - 1;
            }
            const int row0 = off[lo] + (t - start[lo]) * rpt;
            info = int4{lo, row0, min(rpt, off[lo + 1] - row0), 0};
        }
        tile_info[t] = info;
    }
}

hipError_t launch_tile_plan(const int32_t* offsets, int32_t* tile_start, int4* tile_info, int E, int rows_per_tile,
                            int max_tiles, hipStream_t stream) {
    hipLaunchKernelGGL(tile_plan_kernel, dim3(1), dim3(512), 0, stream, offsets, tile_start, tile_info, E,
                       rows_per_tile, max_tiles);
    return hipGetLastError();
}

}  // namespace moe
