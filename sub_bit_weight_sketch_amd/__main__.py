"""``python -m sub_bit_weight_sketch_amd`` builds the HIP library in place."""
from .build import build

if __name__ == "__main__":
    print(build(verbose=True))
