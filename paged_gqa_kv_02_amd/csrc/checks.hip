// checks.hip -- debugging aids, off the hot path.
//  - PGQA_LOG=1: each attention launch prints its route, grid and key split.
//  - pgqa_check_contents: a device-side check of the caller's promises about
//    device array contents (block ids, context lengths, row offsets), which
//    the attention and copy kernels never check (they clamp every index they
//    read instead).  One workgroup per sequence reads that sequence's offsets,
//    length and the block-table entries of the pages a call would touch, and
//    reports violations into a small device status array with vector atomics.
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "device_common.hpp"
#include "launch.hpp"

namespace pgqa {
namespace {

struct CheckArgs {
    const int32_t* block_table;   // [batch, max_blocks_per_seq] or null
    const int32_t* context_lens;  // [batch] or null
    const int32_t* cu;            // [batch + 1] or null
    const int32_t* start_pos;     // [batch] or null (KV write: pages of the written positions)
    int32_t* status;              // [4]: flags, first bad sequence, bad table entries, bad sequences
    int max_blocks_per_seq;
    int batch;
    int total_rows;
    int max_rows;
    int num_blocks;
    int bs_log2;
    int max_context_len;
    int window;
};

__global__ void check_init_kernel(int32_t* status) {
    if (threadIdx.x < 4) status[threadIdx.x] = threadIdx.x == 1 ? INT_MAX : 0;
}

__global__ __launch_bounds__(256) void check_kernel(CheckArgs a) {
    const int b = blockIdx.x;
    int flags = 0;
    // Rows of the sequence (its new tokens): offsets start at 0, never decrease,
    // end at total_rows, and no sequence has more than max_rows.
    // (Contents may be anything: the arithmetic on them is 64-bit.)
    int64_t rows = 0;
    if (a.cu) {
        const int64_t c0 = a.cu[b];
        const int64_t c1 = a.cu[b + 1];
        if ((b == 0 && c0 != 0) || c1 < c0 || (b == a.batch - 1 && c1 != a.total_rows) ||
            (a.max_rows >= 0 && c1 - c0 > a.max_rows))
            flags |= PGQA_CHECK_ROWS;
        rows = c1 > c0 ? c1 - c0 : 0;
    }
    // Positions whose pages the call reads or writes: [p_lo, p_hi).
    int64_t p_lo = 0, p_hi = 0;
    const int64_t table_pos = (int64_t)a.max_blocks_per_seq << a.bs_log2;
    if (a.context_lens) {
        const int64_t L = a.context_lens[b];
        if (L < 0 || L > a.max_context_len) flags |= PGQA_CHECK_CONTEXT;
        const int64_t q = a.cu ? rows : 1;   // without offsets: one query token (decode)
        if (a.cu && L < rows) flags |= PGQA_CHECK_SHORT_CONTEXT;
        if (!a.cu || rows > 0) {
            p_hi = min(min(max(L, (int64_t)0), (int64_t)a.max_context_len), table_pos);
            // Under a window only the first query row's window edge onwards is read.
            if (a.window > 0) p_lo = max((int64_t)0, p_hi - q - a.window + 1);
        }
    } else if (a.start_pos && a.cu) {
        const int64_t s = a.start_pos[b];
        if (s < 0 || s + rows > table_pos) flags |= PGQA_CHECK_CONTEXT;
        p_lo = min(max(s, (int64_t)0), table_pos);
        p_hi = min(max(s, (int64_t)0) + rows, table_pos);
    }
    int bad = 0;
    if (a.block_table && p_hi > p_lo) {
        const int32_t* row = a.block_table + (int64_t)b * a.max_blocks_per_seq;
        const int pg0 = (int)(p_lo >> a.bs_log2);
        const int pg1 = (int)(((p_hi - 1) >> a.bs_log2) + 1);   // <= max_blocks_per_seq
        for (int p = pg0 + (int)threadIdx.x; p < pg1; p += 256) {
            const int id = row[p];
            bad += (id < 0 || id >= a.num_blocks) ? 1 : 0;
        }
    }
    __shared__ int s_bad;
    if (threadIdx.x == 0) s_bad = 0;
    __syncthreads();
    if (bad) atomicAdd(&s_bad, bad);
    __syncthreads();
    if (threadIdx.x != 0) return;
    if (s_bad) flags |= PGQA_CHECK_BLOCK_ID;
    if (!flags) return;
    atomicOr(&a.status[0], flags);
    atomicMin(&a.status[1], b);
    if (s_bad) atomicAdd(&a.status[2], s_bad);
    atomicAdd(&a.status[3], 1);
}

}  // namespace

bool log_enabled() {
    // Read at every launch (a scan of the environment, far below a launch's cost),
    // so a process can switch the log on and off.
    const char* v = std::getenv("PGQA_LOG");
    return v && *v && std::strcmp(v, "0") != 0;
}

void log_line(const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    std::fprintf(stderr, "pgqa: %s\n", buf);
}

hipError_t launch_check(const CheckLaunch& L, hipStream_t stream) {
    hipLaunchKernelGGL(check_init_kernel, dim3(1), dim3(64), 0, stream, L.status);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || L.batch == 0) return err;
    CheckArgs a;
    a.block_table = L.block_table;
    a.context_lens = L.context_lens;
    a.cu = L.cu;
    a.start_pos = L.start_pos;
    a.status = L.status;
    a.max_blocks_per_seq = L.max_blocks_per_seq;
    a.batch = L.batch;
    a.total_rows = L.total_rows;
    a.max_rows = L.max_rows;
    a.num_blocks = L.num_blocks;
    a.bs_log2 = L.block_size_log2;
    a.max_context_len = L.max_context_len;
    a.window = L.window;
    hipLaunchKernelGGL(check_kernel, dim3((unsigned)L.batch), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pgqa
