// Reader of safetensors checkpoint headers (host only).
//
// A safetensors file is an 8-byte little-endian header length N, N bytes of
// JSON mapping each tensor name to {"dtype", "shape", "data_offsets": [begin,
// end]} (plus an optional "__metadata__" object of strings), then the tensor
// bytes, little-endian and row-major, at data_offsets relative to the end of
// the header.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

namespace q3k {

struct StTensor {
  std::string name, dtype;
  std::vector<int64_t> shape;
  uint64_t begin = 0, end = 0;  // byte range within the data section
};

struct StFile {
  std::string path;
  uint64_t data_start = 0;  // file offset of the data section
  std::vector<StTensor> tensors;
};

// Bytes per element of a safetensors dtype name, 0 for an unknown one.
int st_dtype_bytes(const std::string& dtype);

// Parses and checks the header of `path` (offsets inside the file, sizes
// consistent with dtype and shape).  false with *err set on any problem.
bool st_read_header(const std::string& path, StFile* out, std::string* err);

}  // namespace q3k
