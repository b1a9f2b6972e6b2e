// Step 1: block-wise token merging of proxy keys into the compressed store.
//
// Page "Step-5-Preview: Sparse Reads Are Not a Compressed KV Cache":
//   * "Two paths leave the same hidden state" -- proxy keys are LayerNorm'd
//     and carry a 32-dim rotary span; compression logits are a separate
//     projection.
//   * "Eight tokens become one search key, coordinate by coordinate" -- per
//     completed block and per coordinate d, a max-subtracted softmax of the
//     block's logits for d weights the tokens' coordinate d; FP32
//     accumulation; stored through BF16 into E4M3.
//
// Mapping: one wavefront per block (compress_block.hpp), four per
// workgroup.  The kernel streams ~800 B per token at B=8 and is HBM-bound.
#include "compress_block.hpp"

namespace sgqa {
namespace {

using namespace dev;

template <int B>
__global__ __launch_bounds__(256) void compress_kernel(SeqTable seqs, CompressArgs a) {
    const DevSeq sq = seqs.s[blockIdx.y];
    const int64_t r_begin = sq.pos0 / B;
    const int64_t r_end = (sq.pos0 + sq.n_q) / B;
    const int64_t r = r_begin + (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= r_end) return;
    compress_block<B>(sq, r, a);
}

}  // namespace

hipError_t launch_compress(const SeqTable& seqs, int64_t max_blocks, const CompressArgs& a,
                           hipStream_t stream) {
    if (max_blocks <= 0 || seqs.n <= 0) return hipSuccess;
    dim3 grid((unsigned)((max_blocks + 3) / 4), (unsigned)seqs.n);
    dim3 block(256);
    switch (a.block_size) {
        case 1: hipLaunchKernelGGL(compress_kernel<1>, grid, block, 0, stream, seqs, a); break;
        case 2: hipLaunchKernelGGL(compress_kernel<2>, grid, block, 0, stream, seqs, a); break;
        case 4: hipLaunchKernelGGL(compress_kernel<4>, grid, block, 0, stream, seqs, a); break;
        case 8: hipLaunchKernelGGL(compress_kernel<8>, grid, block, 0, stream, seqs, a); break;
        case 16: hipLaunchKernelGGL(compress_kernel<16>, grid, block, 0, stream, seqs, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace sgqa
