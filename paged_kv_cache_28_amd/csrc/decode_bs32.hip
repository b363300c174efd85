// Decode kernels for blocks of 32 tokens (decode_kernels.hpp).
#include "decode_kernels.hpp"

namespace pkv {
template hipError_t dispatch_bs<32>(const DecodeArgs&, int, int, int, dim3, hipStream_t, bool, bool);
}  // namespace pkv
