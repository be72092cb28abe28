// Runs the safetensors header reader of libq3 (decoder_only_qwen3_amd/csrc/
// checkpoint.cpp) over every file named on the command line and prints one
// line per file.  Built by tests/test_sanitizers.py with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host compiler, so a read out of bounds or
// an overflow in the parser of these untrusted files stops the run.
#include <cstdio>
#include <string>

#include "checkpoint.h"

int main(int argc, char** argv) {
  int ok = 0;
  for (int i = 1; i < argc; ++i) {
    q3k::StFile f;
    std::string err;
    if (q3k::st_read_header(argv[i], &f, &err)) {
      ++ok;
      std::printf("ok %zu tensors %s\n", f.tensors.size(), argv[i]);
    } else {
      std::printf("rejected %s: %s\n", argv[i], err.c_str());
    }
  }
  std::printf("%d of %d accepted\n", ok, argc - 1);
  return 0;
}
