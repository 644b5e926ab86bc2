"""The counter tool names every registered micro-kernel as the library
does: its kernel-name parser, applied to the demangled name of each tile
instantiation, gives the registry name (convolution forms: the twin's name
with "_conv")."""
import os
import re

from dynamic_shape_gemm_amd import pmc

SRC = os.path.join(os.path.dirname(pmc.__file__), "csrc", "kernels.hip")


def _registry():
    text = open(SRC).read()
    tiles = {}
    for m in re.finditer(r"using (\w+) = Tile<([^>]*)>;", text):
        args = [a.strip() for a in m.group(2).split(",")]
        args += ["false"] * (9 - len(args))
        tiles[m.group(1)] = ", ".join(args)
    kernels = re.findall(r'MKP_KERNEL\("([^"]+)", (\w+)\)', text)
    convs = re.findall(r'MKP_CONV\("([^"]+)", (\w+)\)', text)
    wsplit = {m.group(1): ", ".join(a.strip() for a in m.group(2).split(","))
              for m in re.finditer(r"using (\w+) = WSplit<([^>]*)>;", text)}
    wkernels = re.findall(r'MKP_WSPLIT\("([^"]+)", (\w+)\)', text)
    return tiles, kernels, convs, wsplit, wkernels


def _demangled(tile_args):
    return (f"void mkp::(anonymous namespace)::gemm_tile_kernel<mkp::(anonymous namespace)::Tile<{tile_args}> >"
            "(mkp::KArgs)")


def test_counter_tool_names_every_kernel():
    tiles, kernels, convs, wsplit, wkernels = _registry()
    assert len(kernels) >= 20 and convs and wkernels
    for name, t in kernels:
        assert pmc.lib_name(_demangled(tiles[t])) == name, (name, tiles[t])
    for twin, t in convs:
        assert pmc.lib_name(_demangled(tiles[t])) == twin + "_conv", (twin, tiles[t])
    for name, w in wkernels:
        demangled = (f"void mkp::(anonymous namespace)::gemm_wsplit_kernel<mkp::(anonymous namespace)::"
                     f"WSplit<{wsplit[w]}> >(mkp::KArgs)")
        assert pmc.lib_name(demangled) == name, (name, wsplit[w])
