// Block, tile and head sizes shared by the host code and the kernels.
#pragma once

namespace bsattn {

constexpr int kBlock = 64;   // tokens per block (b) and per Longformer tile
constexpr int kHead = 64;    // head dimension (d) of every kernel but the d = 128 instances
constexpr int kLfSeg = 8;    // key tiles per work item of a split Longformer global row

}  // namespace bsattn
