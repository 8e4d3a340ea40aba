// KV append for gfx950: writes the qlen newest tokens of every request into
// the paged cache through the block table.
//
// Operation: "Atención paginada", section "Ruta de decodificación" (the
// decode kernel updates the paged cache in place through the block table:
// position j of a request is slot j % P of page block_table[b][j / P]), with
// the position convention of "vllm.models.flint.ops.decode_attention"
// (seq_lens counts the current token, whose K/V is written before the decode
// kernel reads the cache): token t of request b goes to position
// seq_lens[b] - qlen + t.
//
// A byte copy: one lane per 16-byte chunk of a (token, head) row, the chunks
// of the first source followed by those of the second in the cache row.
// Consecutive lanes take consecutive chunks of one row, so both the loads and
// the stores are whole 16-byte vector accesses over contiguous row bytes.
// A token at a negative position, past the block-table row, or behind an
// entry outside [0, num_pages) is not written.
#include "device_common.h"
#include "kernels.h"

namespace pd {
namespace {

__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  const int cpr = a.c0 + a.c1;                       // chunks per (token, head) row
  const int64_t total = (int64_t)a.B * a.qlen * a.H * cpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int chunk = (int)(i % cpr);
    const int64_t rh = i / cpr;
    const int h = (int)(rh % a.H);
    const int64_t row = rh / a.H;                    // b * qlen + t
    const int b = (int)(row / a.qlen), t = (int)(row % a.qlen);
    const int pos = a.seq_lens[b] - a.qlen + t;
    if (pos < 0) continue;
    const int pidx = pos / a.P;
    if (pidx >= a.max_blocks) continue;
    const int page = a.bt[(int64_t)b * a.bt_sb + pidx];
    if (page < 0 || page >= a.num_pages) continue;
    const char* src = chunk < a.c0
                          ? a.src0 + row * a.s0_tok + h * a.s0_h + (int64_t)chunk * 16
                          : a.src1 + row * a.s1_tok + h * a.s1_h + (int64_t)(chunk - a.c0) * 16;
    char* dst = a.cache + (int64_t)page * a.c_sp + (int64_t)h * a.c_sh + (int64_t)(pos % a.P) * a.c_st +
                (int64_t)chunk * 16;
    *(u32x4*)dst = *(const u32x4*)src;
  }
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.B * a.qlen * a.H * (a.c0 + a.c1);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  dim3 grid((unsigned)(blocks < 8192 ? blocks : 8192)), block(256);
  hipLaunchKernelGGL(kv_append_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace pd
